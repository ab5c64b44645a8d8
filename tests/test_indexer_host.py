"""Host side of the pooled indexer, without a GPU: the library's guard decision
(mla_indexer_pool_plan) agrees with the oracle's on every guard, a trim keeps
the incremental path, the selection offsets, and argument errors that are
reported before any device call."""

import ctypes

import numpy as np
import pytest

from mla_speculative_decode_amd import _lib
from oracle import indexer as ix

MLA_OK, MLA_E_NULL, MLA_E_SHAPE, MLA_E_UNSUPPORTED = 0, -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


class HostPool:
    """An mla_pool over host memory: enough for the calls that never launch."""

    def __init__(self, lib, capacity=64, batch_max=4):
        self.buf = np.zeros(16, dtype=np.float32)
        self.lengths = np.zeros(batch_max, dtype=np.int32)
        self.st = _lib.Pool()
        assert lib.mla_indexer_pool_init(ctypes.byref(self.st), self.buf.ctypes.data_as(ctypes.c_void_p), capacity,
                                         batch_max, self.lengths.ctypes.data_as(ctypes.c_void_p)) == MLA_OK

    def pretend_step(self, lengths, d):
        """The state a successful step leaves (the step itself needs a GPU)."""
        self.st.valid, self.st.batch, self.st.d = 1, len(lengths), d
        self.lengths[:len(lengths)] = lengths


def _off(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _plan(lib, pool, lengths_now, S, d, padded=0):
    off = _off(lengths_now)
    inc = ctypes.c_int32(-1)
    st = lib.mla_indexer_pool_plan(ctypes.byref(pool.st), len(lengths_now), d, off.ctypes.data_as(ctypes.c_void_p),
                                   S, padded, ctypes.byref(inc))
    return st, inc.value


def test_init_has_no_pool(lib):
    p = HostPool(lib)
    assert (p.st.valid, p.st.batch, p.st.d) == (0, 0, 0)
    assert _plan(lib, p, [20, 12], 3, 8) == (MLA_OK, 0)


def test_guards_match_the_oracle(lib):
    rng = np.random.default_rng(0)
    for _ in range(400):
        B = int(rng.integers(1, 4))
        d = int(rng.choice([8, 16]))
        prev = [int(x) for x in rng.integers(1, 40, B)]
        S = int(rng.integers(1, 9))
        now = [x + S for x in prev]
        # perturb one thing at random (or nothing)
        kind = int(rng.integers(0, 6))
        p = HostPool(lib)
        state = ix.PoolState()
        if kind != 0:                                     # 0: no pool yet
            p.pretend_step(prev, d)
            state = ix.PoolState(valid=True, batch=B, d=d, lengths=list(prev))
        padded = int(kind == 1)
        d_now = d if kind != 2 else d + 8                 # key width changed
        if kind == 3:                                     # a cache longer than remembered + S
            now[0] += 1
        if kind == 4 and B > 1:                           # batch size changed
            now = now[:-1]
        st, inc = _plan(lib, p, now, S, d_now, padded)
        assert st == MLA_OK
        assert inc == int(ix.guards_hold(state, now, S, d_now, bool(padded))), (kind, prev, now, S)
        assert inc == int(kind == 5 or (kind == 4 and B == 1))


def test_trim_then_append_stays_incremental(lib):
    p = HostPool(lib)
    p.pretend_step([18, 30], 16)
    assert _plan(lib, p, [11, 32], 2, 16) == (MLA_OK, 0)      # cut back without telling the pool
    new = np.array([9, 30], dtype=np.int32)
    assert lib.mla_indexer_pool_trim(ctypes.byref(p.st), 2, new.ctypes.data_as(ctypes.c_void_p)) == MLA_OK
    assert list(p.lengths[:2]) == [9, 30]
    assert _plan(lib, p, [11, 32], 2, 16) == (MLA_OK, 1)
    # a trim never lengthens what the pool covers
    more = np.array([50, 50], dtype=np.int32)
    assert lib.mla_indexer_pool_trim(ctypes.byref(p.st), 2, more.ctypes.data_as(ctypes.c_void_p)) == MLA_OK
    assert list(p.lengths[:2]) == [9, 30]
    bad = np.array([-1, 3], dtype=np.int32)
    assert lib.mla_indexer_pool_trim(ctypes.byref(p.st), 2, bad.ctypes.data_as(ctypes.c_void_p)) == MLA_E_SHAPE
    assert lib.mla_indexer_pool_trim(ctypes.byref(p.st), 1, new.ctypes.data_as(ctypes.c_void_p)) == MLA_E_SHAPE
    q = HostPool(lib)
    assert lib.mla_indexer_pool_trim(ctypes.byref(q.st), 2, new.ctypes.data_as(ctypes.c_void_p)) == MLA_E_SHAPE


def test_selection_offsets(lib):
    lens = [5, 4000, 2048, 1, 2049]
    off = _off(lens)
    out = np.full(len(lens) + 1, -7, dtype=np.int32)
    assert lib.mla_indexer_selection_offsets(len(lens), off.ctypes.data_as(ctypes.c_void_p), 2048,
                                             out.ctypes.data_as(ctypes.c_void_p)) == MLA_OK
    assert list(out) == list(_off([min(2048, x) for x in lens]))
    assert lib.mla_indexer_selection_offsets(len(lens), off.ctypes.data_as(ctypes.c_void_p), 0,
                                             out.ctypes.data_as(ctypes.c_void_p)) == MLA_E_SHAPE


def test_errors_before_any_launch(lib):
    p = HostPool(lib, capacity=8, batch_max=2)
    off = _off([20, 12])
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)   # noqa: E731
    dummy = ctypes.c_void_p(16)   # never dereferenced: every call below fails validation first
    step = lambda B, d, keys, stride, o, S, pool=p: lib.mla_indexer_pool_step(   # noqa: E731
        ctypes.byref(pool.st), B, d, keys, stride, vp(o), dummy, S, 0, None, None)
    assert step(2, 12, dummy, 12, off, 1) == MLA_E_UNSUPPORTED      # d not a multiple of 8
    assert step(2, 1032, dummy, 1032, off, 1) == MLA_E_UNSUPPORTED  # d > 1024
    assert step(2, 16, dummy, 8, off, 1) == MLA_E_SHAPE             # stride < d
    assert step(2, 16, dummy, 16, off, 0) == MLA_E_SHAPE            # S < 1
    assert step(2, 16, dummy, 16, off, 13) == MLA_E_SHAPE           # a cache shorter than S
    assert step(3, 16, dummy, 16, _off([4, 4, 4]), 1) == MLA_E_SHAPE   # more sequences than batch_max
    assert step(2, 16, dummy, 16, _off([40, 12]), 1) == MLA_E_SHAPE    # 10 windows > capacity 8
    assert step(2, 16, None, 16, off, 1) == MLA_E_NULL
    assert p.st.valid == 0
    # the fused step + scores validates the same way, and needs q and scores
    fused = lambda B, d, stride, o, S, q=dummy, sc=dummy, pool=p: lib.mla_indexer_pool_step_scores(   # noqa: E731
        ctypes.byref(pool.st), B, d, dummy, stride, vp(o), dummy, S, 0, q, sc, None, None)
    assert fused(2, 12, 12, off, 1) == MLA_E_UNSUPPORTED
    assert fused(2, 16, 8, off, 1) == MLA_E_SHAPE
    assert fused(2, 16, 16, off, 0) == MLA_E_SHAPE
    assert fused(2, 16, 16, off, 13) == MLA_E_SHAPE
    assert fused(3, 16, 16, _off([4, 4, 4]), 1) == MLA_E_SHAPE
    assert fused(2, 16, 16, _off([40, 12]), 1) == MLA_E_SHAPE
    assert fused(2, 16, 16, off, 1, q=None) == MLA_E_NULL
    assert fused(2, 16, 16, off, 1, sc=None) == MLA_E_NULL
    assert p.st.valid == 0
    # scores need a valid pool that covers the caches as they are
    assert lib.mla_indexer_scores(ctypes.byref(p.st), 2, dummy, vp(off), dummy, dummy, None) == MLA_E_SHAPE
    p.pretend_step([20, 11], 16)
    assert lib.mla_indexer_scores(ctypes.byref(p.st), 2, dummy, vp(off), dummy, dummy, None) == MLA_E_SHAPE
    # selection
    sel = lambda B, cap, o, budget: lib.mla_indexer_select(B, dummy, cap, vp(o), dummy, budget, dummy, dummy,   # noqa: E731
                                                           None)
    assert sel(2, 8, off, 0) == MLA_E_SHAPE
    assert sel(2, 4, off, 16) == MLA_E_SHAPE          # 5 windows > capacity 4
    assert sel(0, 8, off, 16) == MLA_E_SHAPE
    assert lib.mla_indexer_select(2, None, 8, vp(off), dummy, 16, dummy, dummy, None) == MLA_E_NULL


def test_scores_rejected_after_a_trim_inside_a_window(lib):
    """A cut at 9 positions leaves window 2 (positions 8..11) holding the mean of
    rejected rows: scoring before the next step must be refused before any
    launch; a cut on a window boundary leaves every covered window exact."""
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)   # noqa: E731
    dummy = ctypes.c_void_p(16)   # never dereferenced: the calls below fail validation first
    p = HostPool(lib)
    p.pretend_step([12], 16)
    assert lib.mla_indexer_pool_trim(ctypes.byref(p.st), 1, vp(np.array([9], dtype=np.int32))) == MLA_OK
    assert p.st.valid == 2 and list(p.lengths[:1]) == [9]
    assert lib.mla_indexer_scores(ctypes.byref(p.st), 1, dummy, vp(_off([9])), dummy, dummy, None) == MLA_E_SHAPE
    # the stale pool still seeds an incremental step (it recomputes from window 2 on)
    assert _plan(lib, p, [12], 3, 16) == (MLA_OK, 1)
    # a cut on a window boundary: the pool stays scoreable
    q = HostPool(lib)
    q.pretend_step([12], 16)
    assert lib.mla_indexer_pool_trim(ctypes.byref(q.st), 1, vp(np.array([8], dtype=np.int32))) == MLA_OK
    assert q.st.valid == 1
    # (the call then gets past validation and would launch: only its validation is checked here)
    r = HostPool(lib)
    r.pretend_step([12], 16)
    assert lib.mla_indexer_pool_trim(ctypes.byref(r.st), 1, vp(np.array([12], dtype=np.int32))) == MLA_OK
    assert r.st.valid == 1     # nothing was cut


def test_update_list_matches_the_oracle(lib):
    """mla_indexer_update_list against the oracle's fixed-capacity list, over every
    small (first, windows, complete, S, target) and the page's example."""
    import mla_speculative_decode_amd as mla
    assert mla.update_list(6, 8, 8, 5, 8) == [6, 7, 0, 1, 2, 3, 4, 5]      # two real updates, six fillers
    n = 0
    for windows in range(0, 21):
        for complete in range(max(0, windows - 1), windows + 1):          # at most the tail window is partial
            for first in range(0, complete + 1):
                for S in (0, 1, 5, 16, 17):
                    for target in (8, 16):
                        want, C = ix.update_list(list(range(first, windows)), list(range(complete)), target, S,
                                                 fallback=windows - 1)
                        assert mla.update_list(first, windows, complete, S, target) == want, \
                            (first, windows, complete, S, target)
                        n += 1
    assert n > 1000
    out = np.zeros(16, dtype=np.int32)
    cap = ctypes.c_int32()
    vp = out.ctypes.data_as(ctypes.c_void_p)
    assert lib.mla_indexer_update_list(5, 4, 4, 1, 8, vp, ctypes.byref(cap)) == MLA_E_SHAPE   # first > windows
    assert lib.mla_indexer_update_list(0, 4, 5, 1, 8, vp, ctypes.byref(cap)) == MLA_E_SHAPE   # complete > windows
    assert lib.mla_indexer_update_list(0, 4, 4, 1, 12, vp, ctypes.byref(cap)) == MLA_E_SHAPE  # target not 8 / 16
    assert lib.mla_indexer_update_list(0, 4, 4, 1, 8, None, ctypes.byref(cap)) == MLA_E_NULL


def test_fixed_step_validates_before_any_launch(lib):
    p = HostPool(lib, capacity=8, batch_max=2)
    off = _off([20, 12])
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)   # noqa: E731
    dummy = ctypes.c_void_p(16)
    step = lambda S, target, d=16, o=off: lib.mla_indexer_pool_step_fixed(   # noqa: E731
        ctypes.byref(p.st), 2, d, dummy, d, vp(o), dummy, S, 0, target, None, None, None)
    assert step(1, 12) == MLA_E_SHAPE
    assert step(0, 8) == MLA_E_SHAPE
    assert step(1, 8, d=12) == MLA_E_UNSUPPORTED
    assert step(1, 8, o=_off([40, 12])) == MLA_E_SHAPE    # 10 windows > capacity 8
    assert p.st.valid == 0
