"""GPU parity of the fp8 latent cache: mla_quantize_latent_fp8 bit-exact against
the oracle's encoding (codes and power-of-two scales), and the absorbed
attention over the fp8 cache against the oracle's attention over the
dequantised cache (as is the bf16 path fed that dequantised cache: the same
values, summed by another kernel in another order)."""

import math

import numpy as np
import pytest

import oracle
from oracle import fp8
from mla_speculative_decode_amd import synth
from tests.helpers import check_close, dev, host64, sample_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


import mla_speculative_decode_amd as mla  # noqa: E402
from tests.test_parity_gpu import CASES, _inputs  # noqa: E402


def _edge_rows(r, rope):
    """Rows that hit the encoding's corners: all zero, exact midpoints of the
    E4M3 grid (ties to even), the largest value exactly 448 x 2^k, tiny values
    in the subnormal range, negatives that round to zero, large magnitudes."""
    n = r + rope
    v = fp8.decode(np.arange(0x7F))
    mids = (v[:-1] + v[1:]) / 2
    rows = [np.zeros(n)]
    row = np.resize(np.concatenate([mids, -mids]), n)
    row[0] = 448.0
    rows.append(row)                                   # scale 2^0: the midpoints are exact ties
    row = np.resize(np.concatenate([mids, -mids]), n) * 2.0 ** -5
    row[1] = -448.0 * 2.0 ** -5
    rows.append(row)                                   # the same, scaled by 2^-5
    row = np.full(n, -2.0 ** -12)
    row[2] = 1.0
    rows.append(row)                                   # negatives rounding to zero under scale 2^-8
    row = np.linspace(-3e4, 3e4, n)
    rows.append(row)
    row = np.geomspace(1e-6, 1.0, n) * np.where(np.arange(n) % 2, -1, 1)
    rows.append(row)
    x = synth.round_bf16(np.stack(rows).astype(np.float32))
    return x[:, :r], x[:, r:]


@pytest.mark.parametrize("rope", [64, 0])
def test_quantize_bit_exact(rope):
    r = 512
    rng = np.random.default_rng(5)
    T = 1000
    c_kv = synth.round_bf16((rng.standard_normal((T, r)) * np.exp(rng.uniform(-10, 10, (T, 1)))).astype(np.float32))
    k_pe = synth.round_bf16(rng.standard_normal((T, rope)).astype(np.float32))
    ec, ek = _edge_rows(r, rope)
    c_kv = np.concatenate([c_kv, ec])
    k_pe = np.concatenate([k_pe, ek])
    codes, scales = mla.quantize_latent_fp8(dev(c_kv, "bf16"), dev(k_pe, "bf16") if rope else None)
    torch.cuda.synchronize()
    want_codes, want_scales = fp8.quantize_latent(c_kv, k_pe)
    got_codes = codes.cpu().numpy()
    assert np.array_equal(scales.cpu().numpy(), want_scales)
    bad = np.argwhere(got_codes != want_codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


def _fp8_inputs(case):
    x = _inputs(case)
    name, r, n, v, rope, H, L, lens, dt = case
    codes, scales = fp8.quantize_latent(x.c_kv, x.k_pe)
    ch, kh = fp8.dequantize_latent(codes, scales, r)
    return x, codes, scales, ch, kh


@pytest.mark.parametrize("case", [c for c in CASES if c[-1] == "bf16"], ids=[c[0] for c in CASES if c[-1] == "bf16"])
def test_absorbed_fp8_matches_oracle_and_bf16_path(case):
    name, r, n, v, rope, H, L, lens, dt = case
    x, codes, scales, ch, kh = _fp8_inputs(case)
    q_lat = synth.draw_like((len(lens), L, H, r), math.sqrt(n / r), dt, seed=77)
    offs = x.offsets.astype(np.int32)
    c_dev, s_dev = mla.quantize_latent_fp8(dev(x.c_kv, "bf16"), dev(x.k_pe, "bf16") if rope else None)
    ql, qp, wuv = dev(q_lat, "bf16"), dev(x.q_pe, "bf16"), dev(x.w_uv, "bf16")
    out8 = mla.absorbed_attention_fp8(ql, qp, c_dev, s_dev, wuv, offs, scale=x.scale)
    out16 = mla.absorbed_attention(ql, qp, dev(ch.astype(np.float32), "bf16"), dev(kh.astype(np.float32), "bf16"),
                                   wuv, offs, scale=x.scale)
    again = mla.absorbed_attention_fp8(ql, qp, c_dev, s_dev, wuv, offs, scale=x.scale)
    torch.cuda.synchronize()
    assert torch.equal(out8, again), "fp8 path is not deterministic"
    ref = oracle.latent_attention(q_lat, x.q_pe, ch, kh, x.w_uv, x.offsets, L, x.scale)
    check_close(host64(out8).reshape(-1, v), ref, "bf16", f"absorbed fp8 {name}")
    # the bf16 path on the dequantised cache: the same values through kernels that
    # sum in another order, so the same bar rather than the same bits
    check_close(host64(out16).reshape(-1, v), ref, "bf16", f"absorbed bf16 on the dequantised cache {name}")


def test_absorbed_fp8_full_size_sampled():
    w = synth.WORKLOADS["dsv3_h128_kv8192_l8_bf16"]
    x = synth.make_inputs(w)
    codes, scales = fp8.quantize_latent(x.c_kv, x.k_pe)
    ch, kh = fp8.dequantize_latent(codes, scales, w.r)
    d = {k: dev(getattr(x, k), "bf16") for k in ("q_nope", "q_pe", "c_kv", "k_pe", "w_uk", "w_uv")}
    c_dev, s_dev = mla.quantize_latent_fp8(d["c_kv"], d["k_pe"])
    ql = mla.fold_query(d["q_nope"], d["w_uk"])
    out = mla.absorbed_attention_fp8(ql, d["q_pe"], c_dev, s_dev, d["w_uv"], x.offsets.astype(np.int32),
                                     scale=x.scale)
    torch.cuda.synchronize()
    sel = sample_rows(w.batch, x.L, w.heads, 256, seed=11)
    ref = oracle.absorbed(x.q_nope, x.q_pe, ch, kh, x.w_uk, x.w_uv, x.offsets, x.L, x.scale, sel=sel)
    check_close(host64(out).reshape(-1, w.v)[sel], ref, "bf16", "absorbed fp8 full size")


@pytest.mark.parametrize("case,budgets", [
    (("dsv3_sel8", 512, 128, 128, 64, 8, 8, [3000, 700], "bf16"), (512, 300)),
    (("norope_sel8", 512, 128, 128, 0, 8, 4, [1000, 90, 400], "bf16"), (100, 90, 257)),
])
def test_sparse_fp8_matches_oracle_and_sparse_bf16_path(case, budgets):
    """Selected positions over the fp8 cache (and the bf16 selected-position path over the
    dequantised cache): within the bf16 bar of the oracle's attention over the selected
    positions of the dequantised cache."""
    from oracle import sparse
    name, r, n, v, rope, H, L, lens, dt = case
    x, codes, scales, ch, kh = _fp8_inputs(case)
    rng = np.random.default_rng(len(name) + 7)
    sels = [np.sort(np.concatenate([rng.choice(k - 4, size=m - 4, replace=False), np.arange(k - 4, k)]))
            for k, m in zip(lens, budgets)]
    sel = np.concatenate(sels).astype(np.int32)
    soff = np.concatenate([[0], np.cumsum([s.size for s in sels])]).astype(np.int32)
    sel_d = torch.from_numpy(sel).cuda()
    q_lat = synth.draw_like((len(lens), L, H, r), math.sqrt(n / r), dt, seed=78)
    offs = x.offsets.astype(np.int32)
    c_dev, s_dev = mla.quantize_latent_fp8(dev(x.c_kv, "bf16"), dev(x.k_pe, "bf16") if rope else None)
    ql, qp, wuv = dev(q_lat, "bf16"), dev(x.q_pe, "bf16") if rope else None, dev(x.w_uv, "bf16")
    out8 = mla.absorbed_attention_sparse_fp8(ql, qp, c_dev, s_dev, wuv, offs, sel_d, soff, scale=x.scale)
    out16 = mla.absorbed_attention_sparse(ql, qp, dev(ch.astype(np.float32), "bf16"),
                                          dev(kh.astype(np.float32), "bf16") if rope else None, wuv, offs, sel_d,
                                          soff, scale=x.scale)
    again = mla.absorbed_attention_sparse_fp8(ql, qp, c_dev, s_dev, wuv, offs, sel_d, soff, scale=x.scale)
    torch.cuda.synchronize()
    assert torch.equal(out8, again)
    ref = sparse.sparse_latent_attention(q_lat, x.q_pe, ch, kh, x.w_uv, x.offsets, sel, soff, L, x.scale)
    check_close(host64(out8).reshape(-1, v), ref, "bf16", f"sparse fp8 {name}")
    check_close(host64(out16).reshape(-1, v), ref, "bf16", f"sparse bf16 on the dequantised cache {name}")
