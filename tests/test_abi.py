"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, selects paths bit-exactly like the oracle, and rejects bad
arguments on the host before any device call."""

import ctypes
import os
import re

import numpy as np
import pytest

from mla_speculative_decode_amd import _lib
from mla_speculative_decode_amd._lib import Geom
from oracle import threshold as th
from tests.conftest import ROOT


def _header_symbols():
    with open(os.path.join(ROOT, "include", "mla.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\S.*?\b(mla_[a-z0-9_]+)\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    syms = _header_symbols()
    assert len(syms) >= 9
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(_lib.EXPORTS)
    assert lib.mla_version() == 1
    assert lib.mla_status_string(0) == b"ok"
    assert lib.mla_status_string(-4) == b"workspace missing or too small"


def _select(lib, r, n, v, L, T):
    g = Geom(r, n, v, 0, 1)
    p = ctypes.c_int32(-7)
    m = ctypes.c_int64(-7)
    st = lib.mla_select_path(ctypes.byref(g), L, T, ctypes.byref(p), ctypes.byref(m))
    return st, p.value, m.value


def test_select_path_matches_oracle(lib):
    rng = np.random.default_rng(0)
    cases = [(512, 128, 128), (512, 192, 256), (512, 256, 256), (128, 128, 128), (64, 0, 0), (1024, 512, 511),
             (1, 1, 0), (7, 3, 2)]
    cases += [tuple(int(x) for x in rng.integers([1, 0, 0], [2048, 1024, 1024])) for _ in range(300)]
    for (r, n, v) in cases:
        for T in (0, 1, 2, 100, 512, 8192, 32768, 1 << 20, (1 << 31) - 1, 1 << 40):
            m_ref = th.max_absorbed_closed(r, n, v, T)
            for L in {1, 2, 8, m_ref, m_ref + 1, 2048}:
                if T and L > T:
                    continue
                st, p, m = _select(lib, r, n, v, L, T)
                assert st == 0
                assert m == m_ref, (r, n, v, T)
                assert p == th.select_path(r, n, v, L, T)[0]


def test_select_path_printed_values(lib):
    assert _select(lib, 512, 128, 128, 170, 0)[1:] == (0, 170)
    assert _select(lib, 512, 128, 128, 171, 0)[1:] == (1, 170)
    assert _select(lib, 512, 192, 256, 398, 0)[1:] == (0, 398)
    assert _select(lib, 512, 256, 256, 512, 0)[1:] == (0, 512)
    assert _select(lib, 512, 192, 256, 379, 8192)[1:] == (0, 379)
    assert _select(lib, 512, 192, 256, 380, 8192)[1:] == (1, 379)


def test_select_path_errors(lib):
    g = Geom(512, 128, 128, 64, 16)
    p = ctypes.c_int32()
    assert lib.mla_select_path(None, 1, 0, ctypes.byref(p), None) == -1
    assert lib.mla_select_path(ctypes.byref(g), 1, 0, None, None) == -1
    assert lib.mla_select_path(ctypes.byref(g), 0, 0, ctypes.byref(p), None) == -2
    assert lib.mla_select_path(ctypes.byref(g), 1, -1, ctypes.byref(p), None) == -2
    assert lib.mla_select_path(ctypes.byref(g), 9, 8, ctypes.byref(p), None) == -2   # T < L
    assert lib.mla_select_path(ctypes.byref(g), 1, 0, ctypes.byref(p), None) == 0


def _offs(vals):
    a = (ctypes.c_int32 * len(vals))(*vals)
    return a


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def test_workspace_size_and_validation(lib):
    g = Geom(512, 128, 128, 64, 128)
    sz = ctypes.c_size_t()
    off = _offs([0, 8192])
    assert lib.mla_absorbed_workspace_size(ctypes.byref(g), 1, 1, 8, off, ctypes.byref(sz)) == 0
    # 16 splits of 512 positions x 1024 rows: bf16 partial sums (512) + float32 (max, sum)
    assert sz.value == 16 * 1024 * 512 * 2 + 16 * 1024 * 2 * 4
    assert lib.mla_absorbed_workspace_size(ctypes.byref(g), 1, 1, 8, None, ctypes.byref(sz)) == -1
    assert lib.mla_absorbed_workspace_size(ctypes.byref(g), 1, 1, 8, off, None) == -1
    assert lib.mla_absorbed_workspace_size(ctypes.byref(g), 1, 0, 8, off, ctypes.byref(sz)) == -2
    assert lib.mla_absorbed_workspace_size(ctypes.byref(g), 1, 1, 8192 + 1, off, ctypes.byref(sz)) == -2
    assert lib.mla_absorbed_workspace_size(ctypes.byref(g), 7, 1, 8, off, ctypes.byref(sz)) == -3
    bad = Geom(256, 128, 128, 64, 128)
    assert lib.mla_absorbed_workspace_size(ctypes.byref(bad), 1, 1, 8, off, ctypes.byref(sz)) == -3
    # the float32 kernels take other ranks
    assert lib.mla_absorbed_workspace_size(ctypes.byref(bad), 0, 1, 8, off, ctypes.byref(sz)) == 0
    mis = _offs([0, 100, 90])
    assert lib.mla_absorbed_workspace_size(ctypes.byref(g), 1, 2, 4, mis, ctypes.byref(sz)) == -2
    neg = _offs([-1, 100])
    assert lib.mla_absorbed_workspace_size(ctypes.byref(g), 1, 1, 4, neg, ctypes.byref(sz)) == -2
    gm = Geom(1, 192, 256, 64, 32)
    assert lib.mla_materialized_workspace_size(ctypes.byref(gm), 1, 1, 8, off, ctypes.byref(sz)) == 0
    gx = Geom(1, 160, 256, 64, 32)
    assert lib.mla_materialized_workspace_size(ctypes.byref(gx), 1, 1, 8, off, ctypes.byref(sz)) == -3


def test_entry_points_reject_bad_arguments_before_launch(lib):
    g = Geom(512, 128, 128, 64, 16)
    off = _offs([0, 512])
    f = ctypes.c_float(0.07)
    # fold
    assert lib.mla_fold_query(None, 1, 4, FAKE, FAKE, FAKE, None) == -1
    assert lib.mla_fold_query(ctypes.byref(g), 1, 0, FAKE, FAKE, FAKE, None) == -2
    assert lib.mla_fold_query(ctypes.byref(g), 1, 4, None, FAKE, FAKE, None) == -1
    assert lib.mla_fold_query(ctypes.byref(Geom(512, 80, 128, 64, 16)), 1, 4, FAKE, FAKE, FAKE, None) == -3
    # absorbed attention
    args = lambda ws, wsb, **kw: [ctypes.byref(kw.get("g", g)), kw.get("dt", 1), kw.get("B", 1), kw.get("L", 4),
                                  kw.get("ql", FAKE), FAKE, FAKE, FAKE, kw.get("offh", off), FAKE, FAKE, f,
                                  kw.get("out", FAKE), ws, wsb, None]
    assert lib.mla_absorbed_attention(*args(FAKE, 1 << 40, ql=None)) == -1
    assert lib.mla_absorbed_attention(*args(FAKE, 1 << 40, out=None)) == -1
    assert lib.mla_absorbed_attention(*args(FAKE, 1 << 40, offh=None)) == -1
    assert lib.mla_absorbed_attention(*args(FAKE, 1 << 40, L=513)) == -2
    assert lib.mla_absorbed_attention(*args(FAKE, 1 << 40, dt=3)) == -3
    assert lib.mla_absorbed_attention(*args(None, 1 << 40)) == -4
    assert lib.mla_absorbed_attention(*args(FAKE, 16)) == -4
    # materialise
    assert lib.mla_materialize_kv(ctypes.byref(g), 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert lib.mla_materialize_kv(ctypes.byref(g), 1, 16, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.mla_materialize_kv(ctypes.byref(Geom(512, 96, 128, 64, 16)), 1, 16, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, None) == -3
    # materialised attention
    margs = lambda ws, wsb, **kw: [ctypes.byref(kw.get("g", g)), 1, 1, kw.get("L", 4), FAKE, FAKE, FAKE,
                                   kw.get("v", FAKE), off, FAKE, f, FAKE, ws, wsb, None]
    assert lib.mla_materialized_attention(*margs(FAKE, 1 << 40, v=None)) == -1
    assert lib.mla_materialized_attention(*margs(FAKE, 1 << 40, L=600)) == -2
    assert lib.mla_materialized_attention(*margs(FAKE, 0)) == -4
    # selected positions over the bf16 and the fp8 cache: the same checks before any launch
    sel_ok, sel_empty, sel_long = _offs([0, 50]), _offs([0, 0]), _offs([0, 513])
    sargs = lambda soffh, ws, wsb, **kw: [ctypes.byref(g), 1, 4, FAKE, FAKE, kw.get("c", FAKE), FAKE, off, FAKE,
                                          kw.get("sel", FAKE), soffh, FAKE, FAKE, f, FAKE, ws, wsb, None]
    for fn in (lib.mla_absorbed_attention_sparse, lib.mla_absorbed_attention_sparse_fp8):
        assert fn(*sargs(sel_empty, FAKE, 1 << 40)) == -2      # a sequence with nothing selected
        assert fn(*sargs(sel_long, FAKE, 1 << 40)) == -2       # more selected than cached
        assert fn(*sargs(sel_ok, FAKE, 1 << 40, sel=None)) == -1
        assert fn(*sargs(sel_ok, FAKE, 1 << 40, c=None)) == -1
        assert fn(*sargs(sel_ok, None, 1 << 40)) == -4
        assert fn(*sargs(sel_ok, FAKE, 16)) == -4


def test_binding_refuses_cpu_tensors():
    import torch
    import mla_speculative_decode_amd as mla
    x = torch.zeros(1, 2, 128)
    w = torch.zeros(2, 128, 512)
    with pytest.raises(ValueError):
        mla.fold_query(x, w, out=torch.zeros(1, 2, 512))


def test_noalloc_rejects_partials_beyond_its_array(lib):
    # the 32-sequence, 128-head batch plans about 83 MiB of partial results: more
    # than the static array holds, refused before any device call
    import numpy as np
    from mla_speculative_decode_amd import synth
    w = synth.WORKLOADS["dsv3_h128_b32_varlen_l8_bf16"]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    lens = rng.integers(w.kv_range[0], w.kv_range[1], size=w.batch, endpoint=True)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    g = _lib.Geom(512, 128, 128, 64, 128)
    dummy = ctypes.c_void_p(256)
    vp = off.ctypes.data_as(ctypes.c_void_p)
    st = lib.mla_absorbed_attention_noalloc(ctypes.byref(g), _lib.MLA_BF16, w.batch, 8, dummy, dummy, dummy, dummy,
                                            vp, dummy, dummy, ctypes.c_float(0.1), dummy, None)
    assert st == -4   # MLA_E_WORKSPACE
    assert lib.mla_absorbed_attention_noalloc(None, _lib.MLA_BF16, 1, 8, dummy, dummy, dummy, dummy, vp, dummy,
                                              dummy, ctypes.c_float(0.1), dummy, None) == -1


def test_fp8_query_block_entry_points_validate_on_host(lib):
    g = Geom(512, 128, 128, 64, 128)
    sz = ctypes.c_size_t(0)
    assert lib.mla_query_fp8_bytes(ctypes.byref(g), 1, 8, ctypes.byref(sz)) == 0
    assert sz.value == 32 * 19456                       # 1024 rows in tiles of 32
    assert lib.mla_query_fp8_bytes(ctypes.byref(g), 3, 3, ctypes.byref(sz)) == 0
    assert sz.value == 3 * 12 * 19456                   # 384 rows a sequence
    assert lib.mla_query_fp8_bytes(ctypes.byref(g), 0, 8, ctypes.byref(sz)) == -2
    assert lib.mla_query_fp8_bytes(ctypes.byref(g), 1, 8, None) == -1
    d = ctypes.c_void_p(256)
    assert lib.mla_fold_query_fp8(ctypes.byref(g), 1, 8, d, d, None, None, d, None) == -1    # rope > 0, no q_pe
    assert lib.mla_fold_query_fp8(ctypes.byref(g), 1, 8, d, d, d, None, None, None) == -1    # no q8
    assert lib.mla_fold_query_fp8(ctypes.byref(g), 0, 8, d, d, d, None, d, None) == -2
    bad = Geom(256, 128, 128, 64, 128)
    assert lib.mla_fold_query_fp8(ctypes.byref(bad), 1, 8, d, d, d, None, d, None) == -3
    bad = Geom(512, 100, 128, 64, 128)
    assert lib.mla_fold_query_fp8(ctypes.byref(bad), 1, 8, d, d, d, None, d, None) == -3
    off = np.array([0, 64], dtype=np.int32)
    vp = off.ctypes.data_as(ctypes.c_void_p)
    assert lib.mla_absorbed_attention_fp8q(ctypes.byref(g), 1, 8, None, d, d, vp, d, d, ctypes.c_float(0.1), d, d,
                                           1 << 30, None) == -1
    assert lib.mla_absorbed_splits_fp8q(ctypes.byref(g), 1, 8, d, d, d, vp, d, ctypes.c_float(0.1), d, 16,
                                        None) == -4      # workspace too small
