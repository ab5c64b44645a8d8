"""GPU parity of the fp8 latent cache: mla_quantize_latent_fp8 bit-exact against
the oracle's encoding (codes and power-of-two scales), and the absorbed
attention over the fp8 cache, whose scores run on fp8 matrix cores with the
queries quantised to E4M3 in blocks of 32, checked two ways:

* against the oracle's attention of the block-quantised queries (the oracle's
  quantize_query) over the dequantised cache -- the same values, so within the
  bound the path's own bf16 arithmetic implies (helpers.rounding_bound), element
  by element;
* against the oracle's attention over the unquantised queries and cache, within
  the error model's tolerance: |err| <= Z_MAX sigma' per element and the rms of
  err / sigma' at most Z_RMS, where sigma' = sqrt(sigma^2 + (BF16_FLOOR rms)^2)
  joins the model's sigma (oracle fp8.attention_error_sigma: E4M3 rounding of
  queries and cache) and the bf16 rounding of the path's weights and sums."""

import math

import numpy as np
import pytest

import oracle
from oracle import fp8
from mla_speculative_decode_amd import synth
from tests.helpers import check_close, check_within, dev, host64, rounding_bound, sample_rows

# Error-model gate.  sigma is a standard deviation of a sum of many small
# independent roundings, near normal: 6 sigma is exceeded with probability
# 2e-9 per element under the model, and the model matches sampled E4M3 rounding
# within 10 % in variance (the oracle's Monte Carlo pin), so an rms of
# err / sigma' above 1.5 means errors the model does not explain.  BF16_FLOOR:
# the bf16 rounding of P, of the split partials and of W_UV's product (a few
# units of 2^-9 relative each) as a fraction of the output rms.
Z_MAX = 6.0
Z_RMS = 1.5
BF16_FLOOR = 2.0 ** -8


def _qq(q):
    """The block-quantised queries the fp8 path scores with (oracle)."""
    q = np.asarray(q)
    return fp8.quantize_query(q)[0] if q.shape[-1] else q.astype(np.float64)


def _gate(got, exact, sigma, what):
    rms = float(np.sqrt(np.mean(exact * exact)))
    tol = np.sqrt(sigma * sigma + (BF16_FLOOR * rms) ** 2)
    z = np.abs(got - exact) / tol
    zmax, zrms = float(z.max()), float(np.sqrt(np.mean(z * z)))
    rel = float(np.sqrt(np.mean((got - exact) ** 2))) / rms
    print(f"{what}: rms err / rms out {rel:.4f}, model sigma rms / rms out "
          f"{float(np.sqrt(np.mean(sigma ** 2))) / rms:.4f}, max z {zmax:.2f}, rms z {zrms:.3f}", flush=True)
    assert zmax <= Z_MAX, f"{what}: max |err| / sigma' = {zmax:.2f} > {Z_MAX}"
    assert zrms <= Z_RMS, f"{what}: rms err / sigma' = {zrms:.3f} > {Z_RMS}"

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
def test_absorbed_fp8_matches_oracle(case):
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
    got = host64(out8).reshape(-1, v)
    qlq, qpq = _qq(q_lat), _qq(x.q_pe)
    ref_q = oracle.latent_attention(qlq, qpq, ch, kh, x.w_uv, x.offsets, L, x.scale)
    allr = np.arange(got.shape[0])
    bound = rounding_bound(qlq, qpq, ch, kh, x.w_uv, x.offsets, L, x.scale, allr)
    worst = check_within(got, ref_q, bound, f"absorbed fp8 {name} (block-quantised queries, dequantised cache)")
    print(f"absorbed fp8 {name}: max |err| / rounding bound {worst:.3f}", flush=True)
    # the bf16 path on the dequantised cache (unquantised queries)
    ref = oracle.latent_attention(q_lat, x.q_pe, ch, kh, x.w_uv, x.offsets, L, x.scale)
    check_close(host64(out16).reshape(-1, v), ref, "bf16", f"absorbed bf16 on the dequantised cache {name}")
    # against the unquantised inputs, within the error model
    rows = sample_rows(len(lens), L, H, 40, seed=len(name))
    exact = oracle.latent_attention(q_lat, x.q_pe, x.c_kv, x.k_pe, x.w_uv, x.offsets, L, x.scale, sel=rows)
    sigma = fp8.attention_error_sigma(q_lat, x.q_pe, x.c_kv, x.k_pe, x.w_uv, x.offsets, L, x.scale, rows)
    _gate(got[rows], exact, sigma, f"absorbed fp8 {name} vs unquantised")


def test_absorbed_fp8_full_size_sampled():
    """The headline workload (128 heads, 8 rows per verify block, 8192 cached
    positions) in the launch configuration the benchmark times: sampled rows
    against the oracle, both ways."""
    w = synth.WORKLOADS["dsv3_h128_kv8192_l8_bf16"]
    x = synth.make_inputs(w)
    codes, scales = fp8.quantize_latent(x.c_kv, x.k_pe)
    ch, kh = fp8.dequantize_latent(codes, scales, w.r)
    q_lat = synth.draw_like((w.batch, x.L, w.heads, w.r), math.sqrt(w.n / w.r), "bf16", seed=79)
    d = {k: dev(getattr(x, k), "bf16") for k in ("q_pe", "c_kv", "k_pe", "w_uv")}
    c_dev, s_dev = mla.quantize_latent_fp8(d["c_kv"], d["k_pe"])
    out = mla.absorbed_attention_fp8(dev(q_lat, "bf16"), d["q_pe"], c_dev, s_dev, d["w_uv"],
                                     x.offsets.astype(np.int32), scale=x.scale)
    torch.cuda.synchronize()
    got = host64(out).reshape(-1, w.v)
    sel = sample_rows(w.batch, x.L, w.heads, 256, seed=11)
    qlq, qpq = _qq(q_lat), _qq(x.q_pe)
    ref = oracle.latent_attention(qlq, qpq, ch, kh, x.w_uv, x.offsets, x.L, x.scale, sel=sel)
    bound = rounding_bound(qlq, qpq, ch, kh, x.w_uv, x.offsets, x.L, x.scale, sel)
    worst = check_within(got[sel], ref, bound, "absorbed fp8 full size (block-quantised queries, dequantised cache)")
    print(f"absorbed fp8 full size: max |err| / rounding bound {worst:.3f}", flush=True)
    rows = sel[:: max(1, len(sel) // 12)]
    exact = oracle.latent_attention(q_lat, x.q_pe, x.c_kv, x.k_pe, x.w_uv, x.offsets, x.L, x.scale, sel=rows)
    sigma = fp8.attention_error_sigma(q_lat, x.q_pe, x.c_kv, x.k_pe, x.w_uv, x.offsets, x.L, x.scale, rows)
    _gate(got[rows], exact, sigma, "absorbed fp8 full size vs unquantised")


@pytest.mark.parametrize("case,budgets", [
    (("dsv3_sel8", 512, 128, 128, 64, 8, 8, [3000, 700], "bf16"), (512, 300)),
    (("norope_sel8", 512, 128, 128, 0, 8, 4, [1000, 90, 400], "bf16"), (100, 90, 257)),
])
def test_sparse_fp8_matches_oracle_and_sparse_bf16_path(case, budgets):
    """Selected positions over the fp8 cache: within the bf16 bar of the oracle's
    attention of the block-quantised queries over the selected positions of the
    dequantised cache (and the bf16 selected-position path over that cache
    within the bar of the oracle with unquantised queries)."""
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
    ref_q = sparse.sparse_latent_attention(_qq(q_lat), _qq(x.q_pe), ch, kh, x.w_uv, x.offsets, sel, soff, L, x.scale)
    check_close(host64(out8).reshape(-1, v), ref_q, "bf16", f"sparse fp8 {name}")
    ref = sparse.sparse_latent_attention(q_lat, x.q_pe, ch, kh, x.w_uv, x.offsets, sel, soff, L, x.scale)
    check_close(host64(out16).reshape(-1, v), ref, "bf16", f"sparse bf16 on the dequantised cache {name}")
