"""Pins of the pooled-indexer oracle ("One guard, 110x off the verify step",
section "The same bug, one layer over"): closed forms of the window mean, the
pages' own check that a wide step pools exactly as the same tokens fed one at a
time (two, three, four and eight new tokens at aligned and misaligned lengths),
each guard forcing a full recompute, a pool that trusts its remembered length
without the length guard going stale after a trim, and the selection against
independent constructions (top windows by argsort, ties, partial windows)."""

import numpy as np
import pytest

from oracle import indexer as ix


def _keys(T, d=6, seed=0):
    return np.random.default_rng(seed).standard_normal((T, d))


def test_window_mean_closed_form():
    # key row t = (t, -2t, 1): a full window w pools to 4w + 1.5; a tail window of
    # n rows to 4w + (n - 1) / 2
    for T in (1, 2, 3, 4, 5, 11, 16):
        keys = np.stack([np.array([t, -2.0 * t, 1.0]) for t in range(T)])
        P = ix.pool_all(keys, T)
        assert P.shape == (ix.n_windows(T), 3)
        for w in range(P.shape[0]):
            n = min(4, T - 4 * w)
            c = 4 * w + (n - 1) / 2
            assert np.allclose(P[w], [c, -2 * c, 1.0], rtol=0, atol=1e-12)


def test_constant_rows_pool_to_themselves():
    # catches a tail window divided by 4 instead of by its row count
    for T in (5, 6, 7):
        P = ix.pool_all(np.full((T, 4), 3.25), T)
        assert np.all(P == 3.25)


@pytest.mark.parametrize("T0", [16, 17, 18, 19])
@pytest.mark.parametrize("S", [2, 3, 4, 8])
def test_wide_step_equals_one_at_a_time(T0, S):
    keys = _keys(T0 + S, seed=T0 * 10 + S)
    wide, narrow = ix.PoolState(), ix.PoolState()
    assert not ix.pool_step(wide, [keys[:T0]], S=T0)          # no pool yet: full
    assert not ix.pool_step(narrow, [keys[:T0]], S=T0)
    assert ix.pool_step(wide, [keys[:T0 + S]], S=S)            # guards hold: tail only
    for k in range(1, S + 1):
        assert ix.pool_step(narrow, [keys[:T0 + k]], S=1)
    assert wide.lengths == narrow.lengths == [T0 + S]
    Pw, Pn = ix.pooled_array(wide, 0), ix.pooled_array(narrow, 0)
    ref = ix.pool_all(keys, T0 + S)
    assert np.array_equal(Pw, Pn)
    assert np.allclose(Pw, ref, rtol=0, atol=1e-12)
    q = np.random.default_rng(1).standard_normal(keys.shape[1])
    for budget in (4, 6, 9):
        sw = ix.select_positions(ix.window_scores(Pw, q), T0 + S, budget)
        sn = ix.select_positions(ix.window_scores(Pn, q), T0 + S, budget)
        assert np.array_equal(sw, sn)


def test_each_guard_forces_a_full_recompute():
    keys = _keys(40, d=5)
    base = ix.PoolState()
    ix.pool_step(base, [keys[:20], keys[:12]], S=20)

    def fresh():
        st = ix.PoolState(valid=base.valid, batch=base.batch, d=base.d, lengths=list(base.lengths),
                          pooled=[dict(p) for p in base.pooled])
        return st

    assert ix.pool_step(fresh(), [keys[:23], keys[:15]], S=3)                      # all guards hold
    assert not ix.pool_step(ix.PoolState(), [keys[:23], keys[:15]], S=3)           # no pool
    assert not ix.pool_step(fresh(), [keys[:23], keys[:15]], S=3, padded=True)     # padding
    assert not ix.pool_step(fresh(), [keys[:23]], S=3)                              # batch size changed
    assert not ix.pool_step(fresh(), [keys[:23, :4], keys[:15, :4]], S=3)          # key width changed
    assert not ix.pool_step(fresh(), [keys[:24], keys[:15]], S=3)                  # length not remembered
    # whichever path ran, the pool is the definition
    st = fresh()
    ix.pool_step(st, [keys[:24], keys[:15]], S=3)
    assert np.allclose(ix.pooled_array(st, 0), ix.pool_all(keys, 24), rtol=0, atol=1e-12)
    assert np.allclose(ix.pooled_array(st, 1), ix.pool_all(keys, 15), rtol=0, atol=1e-12)


def _trusting_step(state, keys, S):
    """Planted mistake: an incremental step that trusts the pool's remembered
    length (recomputes from the window it last left open) and has no length guard."""
    T = len(keys)
    first = state.lengths[0] // ix.WINDOW
    for w in range(first, ix.n_windows(T)):
        state.pooled[0][w] = ix.pool_window(keys, w, T)
    state.lengths = [T]


def test_trim_needs_the_length_guard():
    # 18 positions pooled, a rejection cuts the cache back to 9, two new tokens
    # arrive: positions 9 and 10 now hold different keys than the pool saw
    old = _keys(18, seed=5)
    new = np.concatenate([old[:9], _keys(2, seed=6)])
    st = ix.PoolState()
    ix.pool_step(st, [old], S=18)
    stale = ix.PoolState(valid=True, batch=1, d=old.shape[1], lengths=[18], pooled=[dict(st.pooled[0])])
    _trusting_step(stale, new, S=2)
    P_stale = np.stack([stale.pooled[0][w] for w in range(ix.n_windows(11))])
    ref = ix.pool_all(new, 11)
    assert not np.allclose(P_stale, ref)                   # window 2 still pools rejected keys
    assert not ix.pool_step(st, [new], S=2)                # the guard sees 18 != 11 - 2
    assert np.allclose(ix.pooled_array(st, 0), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("trim_to", [8, 9, 11])
def test_announced_trim_keeps_the_incremental_path(trim_to):
    old = _keys(18, seed=7)
    new = np.concatenate([old[:trim_to], _keys(3, seed=8)])
    st = ix.PoolState()
    ix.pool_step(st, [old], S=18)
    ix.pool_trim(st, [trim_to])
    assert st.lengths == [trim_to]
    assert ix.pool_step(st, [new], S=3)
    assert np.allclose(ix.pooled_array(st, 0), ix.pool_all(new, trim_to + 3), rtol=0, atol=1e-12)


def test_scores_pick_columns_and_are_linear():
    P = ix.pool_all(_keys(13, d=7, seed=2), 13)
    for j in range(7):
        e = np.zeros(7)
        e[j] = 1.0
        assert np.array_equal(ix.window_scores(P, e), P[:, j])
    a, b = np.arange(7.0), np.ones(7)
    assert np.allclose(ix.window_scores(P, 2 * a - b), 2 * ix.window_scores(P, a) - ix.window_scores(P, b),
                       rtol=0, atol=1e-12)


def test_selection_short_cache_takes_everything():
    assert np.array_equal(ix.select_positions([0.3, -1.0, 2.0], 10, 16), np.arange(10))
    assert np.array_equal(ix.select_positions([0.3, -1.0, 2.0], 10, 10), np.arange(10))


def test_selection_is_the_top_windows():
    rng = np.random.default_rng(3)
    T, budget = 400, 64
    s = rng.permutation(100).astype(float)          # distinct window scores
    top = np.argsort(-s)[:budget // 4]
    ref = np.sort(np.concatenate([np.arange(4 * w, 4 * w + 4) for w in top]))
    assert np.array_equal(ix.select_positions(s, T, budget), ref)


def test_selection_ties_and_partial_windows():
    # all equal: the lowest positions
    assert np.array_equal(ix.select_positions(np.zeros(5), 20, 7), np.arange(7))
    # -0 and +0 are equal scores
    assert np.array_equal(ix.select_positions([-0.0, 0.0, -1.0], 12, 6), np.arange(6))
    # boundary window cut: best window 3 whole, then the two lowest positions of window 1
    assert np.array_equal(ix.select_positions([0.0, 5.0, 1.0, 9.0], 16, 6), [4, 5, 12, 13, 14, 15])
    # the tail window holds 2 positions (T = 10): it is taken whole, then 2 of the next
    assert np.array_equal(ix.select_positions([1.0, 0.5, 7.0], 10, 4), [0, 1, 8, 9])


def test_selection_invariants_random():
    rng = np.random.default_rng(4)
    for _ in range(50):
        T = int(rng.integers(1, 300))
        budget = int(rng.integers(1, 80))
        W = ix.n_windows(T)
        s = np.round(rng.standard_normal(W), 1)     # many ties
        sel = ix.select_positions(s, T, budget)
        assert sel.size == min(budget, T)
        assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < T
        rest = np.setdiff1d(np.arange(T), sel)
        if rest.size and sel.size:
            worst_in = min(s[sel // 4])
            best_out = max(s[rest // 4])
            assert worst_in >= best_out
            # among positions of the threshold score, the selected ones come first
            tied_in = sel[s[sel // 4] == worst_in]
            tied_out = rest[s[rest // 4] == worst_in]
            if tied_out.size:
                assert tied_in.max() < tied_out.min()


# ---- fixed-capacity update list ------------------------------------------------

def _golden_lists():
    from tests.conftest import golden_path
    out = []
    with open(golden_path("pad8_update_list.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, delta, complete, P, m, want, C = [x.strip() for x in line.split("|")]
            ints = lambda s: [] if s == "-" else [int(v) for v in s.split(",")]   # noqa: E731
            out.append((name, ints(delta), ints(complete), int(P), int(m), ints(want), int(C)))
    return out


@pytest.mark.parametrize("case", _golden_lists(), ids=lambda c: c[0])
def test_update_list_matches_the_page(case):
    name, delta, complete, P, m, want, C = case
    assert ix.update_list(delta, complete, P, m) == (want, C)


def test_update_list_without_anything_uses_the_fallback():
    assert ix.update_list([], [], 8, 1, fallback="fb") == (["fb"], 1)
    # padding off: the list keeps its size
    assert ix.update_list([5, 6], list(range(10)), 8, 2, padding=False) == ([5, 6], 2)


def test_update_list_invariants_on_random_steps():
    rng = np.random.default_rng(17)
    for _ in range(2000):
        T = int(rng.integers(1, 200))
        S = int(rng.integers(1, min(T, 24) + 1))
        P = int(rng.choice([8, 16]))
        delta = list(range((T - S) // ix.WINDOW, ix.n_windows(T)))
        complete = list(range(T // ix.WINDOW))
        U, C = ix.update_list(delta, complete, P, S)
        assert len(U) == C and U[:len(delta)] == delta            # every real update is kept, first
        assert len(set(U)) == len(U)                               # distinct destinations
        assert all(u in complete for u in U[len(delta):])          # fillers are complete windows
        padded = S <= 16 and len(delta) <= P and len(complete) >= P
        assert C == (P if padded else len(delta))


def test_fixed_step_pools_like_the_variable_step():
    # the same step sequence through pool_step and pool_step_fixed: identical
    # pooled keys (the fillers' writes reproduce the stored values exactly)
    rng = np.random.default_rng(23)
    d = 6
    total = 160
    keys = rng.standard_normal((total, d))
    a, f = ix.PoolState(), ix.PoolState()
    T = 40
    ix.pool_step(a, [keys[:T]], T)
    ix.pool_step_fixed(f, [keys[:T]], T)
    padded_steps = 0
    for S in [1, 3, 5, 2, 8, 4, 7, 1, 16, 6, 9, 20]:
        T += S
        stored = {w: v.copy() for w, v in f.pooled[0].items()}
        ia = ix.pool_step(a, [keys[:T]], S)
        inc, lists = ix.pool_step_fixed(f, [keys[:T]], S)
        assert ia and inc
        U = lists[0]
        padded_steps += len(U) == 8
        for w in U:
            if w < (T - S) // ix.WINDOW:      # a filler: its value is unchanged, bit for bit
                assert np.array_equal(f.pooled[0][w], stored[w])
        assert np.array_equal(ix.pooled_array(a, 0), ix.pooled_array(f, 0))
    assert padded_steps == 11                  # every step pads but the last: 20 tokens > 16 keep their 6 windows
