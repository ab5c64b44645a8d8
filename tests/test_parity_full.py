"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (fold, then split-KV pass, then merge), checked against the
float64 oracle on every (row, head) pair where it finishes in seconds (the
one-sequence workloads) and on sampled pairs that it computes one by one
elsewhere (the 32-sequence batch).

Workloads: DeepSeek-V3 geometry 16 heads / Kv 512 / L 4 in float32 (both
paths, every row); 128 heads / Kv 8192 / L 8 bf16; GLM-4.7-Flash-like 32 heads
/ Kv 8192 with L swept over 1..2048 and each path forced; GLM-5.3-Flash-like
64 heads / Kv 32768 / L 16; 32 sequences with Kv ~ U[1024, 32768], L 8.
"""

import numpy as np
import pytest

import oracle
from mla_speculative_decode_amd import synth
from tests.helpers import check_close, host64, sample_rows

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


import mla_speculative_decode_amd as mla  # noqa: E402

_cache = {}


def _load(name, L=None):
    key = (name, L)
    if key not in _cache:
        _cache.clear()
        w = synth.WORKLOADS[name]
        x = synth.make_inputs(w, L=L)
        dt = w.dtype
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        d = {k: torch.from_numpy(getattr(x, k)).to(tdt).to("cuda") for k in
             ("q_nope", "q_pe", "c_kv", "k_pe", "w_uk", "w_uv")}
        _cache[key] = (x, d, mla.Offsets(x.offsets.astype(np.int32), "cuda"))
    return _cache[key]


def _absorbed(d, offs, x):
    out = mla.absorbed(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"], offs, scale=x.scale)
    torch.cuda.synchronize()
    return host64(out).reshape(-1, x.w.v)


def _ref_rows(x, sel):
    return oracle.absorbed(x.q_nope, x.q_pe, x.c_kv, x.k_pe, x.w_uk, x.w_uv, x.offsets, x.L, x.scale, sel=sel)


def test_dsv3_f32_both_paths_all_rows():
    x, d, offs = _load("dsv3_h16_kv512_l4_f32")
    ref = oracle.absorbed(x.q_nope, x.q_pe, x.c_kv, x.k_pe, x.w_uk, x.w_uv, x.offsets, x.L, x.scale)
    check_close(_absorbed(d, offs, x), ref, "f32", "absorbed f32")
    m = mla.materialized(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"], offs, scale=x.scale)
    torch.cuda.synchronize()
    check_close(host64(m).reshape(ref.shape), ref, "f32", "materialized f32")
    mref = oracle.materialized(x.q_nope, x.q_pe, x.c_kv, x.k_pe, x.w_uk, x.w_uv, x.offsets, x.L, x.scale)
    assert np.max(np.abs(mref - ref)) <= 1e-12


@pytest.mark.parametrize("name,all_rows", [("dsv3_h128_kv8192_l8_bf16", True), ("glm53_h64_kv32768_l16_bf16", True),
                                           ("dsv3_h128_b32_varlen_l8_bf16", False),
                                           ("dsv3_h16_kv8192_l8_bf16", True), ("dsv3_h16_b32_varlen_l8_bf16", False)])
def test_absorbed_full_size(name, all_rows):
    x, d, offs = _load(name)
    got = _absorbed(d, offs, x)
    assert np.all(np.isfinite(got))
    if all_rows:
        check_close(got, _ref_rows(x, None), "bf16", f"absorbed {name} (every row)")
    else:
        sel = sample_rows(x.w.batch, x.L, x.w.heads, 192, seed=1)
        check_close(got[sel], _ref_rows(x, sel), "bf16", f"absorbed {name}")
    # the split pass + merge through the separate entry points gives the same bits
    geom = mla.Geom(x.w.r, x.w.n, x.w.v, x.w.rope, x.w.heads)
    ws = torch.empty(mla.absorbed_workspace_size(geom, 1, x.L, offs), dtype=torch.uint8, device="cuda")
    ql = mla.fold_query(d["q_nope"], d["w_uk"])
    mla.absorbed_splits(ql, d["q_pe"], d["c_kv"], d["k_pe"], offs, geom, x.scale, ws)
    out = torch.empty((x.w.batch, x.L, x.w.heads, x.w.v), dtype=torch.float32, device="cuda")
    mla.absorbed_merge(d["w_uv"], out, offs, geom, x.L, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host64(out).reshape(-1, x.w.v), got)


@pytest.mark.parametrize("L", synth.SWEEP_L)
def test_glm47_sweep_both_paths_sampled(L):
    x, d, offs = _load("glm47_h32_kv8192_bf16", L=L)
    sel = sample_rows(1, L, x.w.heads, 128, seed=L)
    ref = _ref_rows(x, sel)
    got_a = _absorbed(d, offs, x)
    check_close(got_a[sel], ref, "bf16", f"absorbed L={L}")
    m = mla.materialized(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"], offs, scale=x.scale)
    torch.cuda.synchronize()
    got_m = host64(m).reshape(-1, x.w.v)
    # bf16 storage of the expanded K and V: bar derived in test_parity_gpu.test_materialized_chain
    check_close(got_m[sel], ref, "bf16", f"materialized L={L}", rel=4e-2)
    g = mla.Geom(512, 192, 256, 64, 32)
    path, m_abs = mla.select_path(g, L, 8192)
    assert m_abs == 379 and path == (mla.MLA_ABSORBED if L <= 379 else mla.MLA_MATERIALIZED)
