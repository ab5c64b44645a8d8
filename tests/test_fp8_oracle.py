"""Pins of the fp8 (OCP E4M3) latent-cache oracle against the format's own
definition: the value table, round-to-nearest-even at every midpoint,
saturation, the power-of-two row scale, and the dequantisation error bound."""

import numpy as np
import pytest

from oracle import fp8
from mla_speculative_decode_amd import synth


def test_value_table_anchors():
    v = fp8.decode(np.arange(256))
    # zero, smallest subnormal, largest subnormal, smallest normal, one, largest finite
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x7E] == 448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.all(v[0x80:0xFF] == -v[0x00:0x7F])
    assert np.all(np.diff(v[0x00:0x7F]) > 0)          # codes 0x00..0x7e are strictly increasing
    # the spacing doubles at every binade: 2^(e-10) in binade e >= 1 (and 2^-9 below)
    for e in range(1, 16):
        codes = np.arange(8 * e, 8 * e + 8)
        codes = codes[codes <= 0x7E]
        assert np.allclose(np.diff(v[codes]), 2.0 ** (e - 10))


def test_encode_inverts_decode():
    c = np.arange(0x7F)
    assert np.array_equal(fp8.encode(fp8.decode(c)), c)
    assert np.array_equal(fp8.encode(-fp8.decode(c[1:])), c[1:] | 0x80)
    assert fp8.encode(np.array([-0.0]))[0] == 0x00


def test_round_to_nearest_even_at_midpoints():
    v = fp8.decode(np.arange(0x7F))
    mid = (v[:-1] + v[1:]) / 2
    got = fp8.encode(mid)
    lo, hi = np.arange(0x7E), np.arange(1, 0x7F)
    want = np.where(lo % 2 == 0, lo, hi)              # the even code of the two neighbours
    assert np.array_equal(got, want)
    eps = np.minimum(np.diff(v) * 1e-3, 1e-12)
    assert np.array_equal(fp8.encode(mid + eps), hi)
    assert np.array_equal(fp8.encode(mid - eps), lo)


def test_saturation():
    assert fp8.encode(np.array([448.0, 460.0, 1e9]))[0] == 0x7E
    assert np.all(fp8.encode(np.array([460.0, 1e9])) == 0x7E)
    assert np.all(fp8.encode(np.array([-460.0, -1e9])) == 0xFE)


def test_row_scale_is_the_smallest_power_of_two():
    rng = np.random.default_rng(0)
    amax = np.concatenate([np.exp(rng.uniform(-30, 30, 2000)), [448.0, 224.0, 1.0, 3.5, 3.5000001]])
    k = fp8.row_scale_exponent(amax)
    assert np.all(448.0 * np.exp2(k.astype(float)) >= amax)
    assert np.all(448.0 * np.exp2(k.astype(float) - 1) < amax)
    assert list(fp8.row_scale_exponent(np.array([0.0, 448.0, 224.0, 1.0]))) == [0, 0, -1, -8]


def test_quantize_error_bound_and_bf16_exactness():
    rng = np.random.default_rng(1)
    T, r, rope = 300, 512, 64
    c_kv = synth.round_bf16((rng.standard_normal((T, r)) * np.exp(rng.uniform(-8, 8, (T, 1)))).astype(np.float32))
    k_pe = synth.round_bf16(rng.standard_normal((T, rope)).astype(np.float32))
    c_kv[3] = 0.0
    k_pe[3] = 0.0
    codes, scales = fp8.quantize_latent(c_kv, k_pe)
    assert codes.shape == (T, r + rope) and codes.dtype == np.uint8 and scales.dtype == np.float32
    assert scales[3] == 1.0 and np.all(codes[3] == 0)
    ch, kh = fp8.dequantize_latent(codes, scales, r)
    x = np.concatenate([c_kv, k_pe], axis=1).astype(np.float64)
    xh = np.concatenate([ch, kh], axis=1)
    s = scales.astype(np.float64)[:, None]
    y = np.abs(x) / s
    # half a spacing: relative 2^-4 on the normal grid, 2^-10 x scale below it
    bound = np.where(y >= 2.0 ** -6, np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s)
    assert np.all(np.abs(xh - x) <= bound * (1 + 1e-12))
    # each nonzero row's largest magnitude is in (224, 448] x scale before rounding,
    # [224, 448] x scale after (values just above 224 round down to it)
    nz = np.max(np.abs(x), axis=1) > 0
    amax_y = np.max(np.abs(x), axis=1)[nz] / scales[nz]
    amax_code = np.max(np.abs(xh), axis=1)[nz] / scales[nz]
    assert np.all((amax_y > 224) & (amax_y <= 448))
    assert np.all((amax_code >= 224) & (amax_code <= 448))
    # dequantised values are exact in bfloat16
    assert np.array_equal(synth.round_bf16(xh.astype(np.float32)).astype(np.float64), xh)


def test_query_blocks_are_cache_rows_of_32():
    """quantize_query on a row is quantize_latent on each 32-wide block of it taken
    as a cache row of its own (the blocks do not share a scale): one huge block
    does not coarsen its neighbours."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((5, 128)) * np.exp(rng.uniform(-6, 6, (5, 1)))
    q[1, 40] = 3e4                     # block 1 of row 1 only
    q[2, :32] = 0.0                    # an all-zero block: scale 2^0, codes 0
    deq, codes, k = fp8.quantize_query(q)
    for row in range(q.shape[0]):
        for j in range(4):
            blk = q[row, 32 * j:32 * j + 32][None, :]
            c, s = fp8.quantize_latent(blk, np.zeros((1, 0)))
            assert np.array_equal(codes[row, 32 * j:32 * j + 32], c[0])
            assert 2.0 ** k[row, j] == s[0]
    assert k[1, 1] > k[1, 0] + 10 and k[1, 2] == fp8.row_scale_exponent(np.max(np.abs(q[1, 64:96])))
    assert np.all(codes[2, :32] == 0) and k[2, 0] == 0
    # within half a step of the E4M3 grid (2^-4 relative in the normal range)
    y = np.abs(q) * np.exp2(-np.repeat(k, 32, axis=1))
    normal = y >= 2.0 ** -6
    assert np.all(np.abs(deq - q)[normal] <= np.abs(q)[normal] * 2.0 ** -4 + 1e-300)


def _mc_problem(aligned: bool = False):
    """A small problem; `aligned` gives W_UV columns a large component along the
    rows' queries, which makes the cross term of the cache part (a key error and
    the same value error) large: a wrong sign there then fails the pin."""
    rng = np.random.default_rng(17)
    B, L, H, r, rope, v, T = 1, 2, 2, 64, 32, 32, 300
    q_lat = rng.standard_normal((B, L, H, r))
    q_pe = rng.standard_normal((B, L, H, rope))
    c_kv = rng.standard_normal((T, r)) * np.exp(rng.uniform(-1, 1, (T, 1)))
    k_pe = rng.standard_normal((T, rope))
    w_uv = rng.standard_normal((H, r, v)) / np.sqrt(r)
    offsets = np.array([0, T], dtype=np.int64)
    if aligned:
        sign = np.where(np.arange(v) % 2, 1.0, -1.0)
        for h in range(H):
            u = q_lat[0, :, h].mean(axis=0)
            w_uv[h] = 0.3 * w_uv[h] + 2.0 * (u / np.linalg.norm(u))[:, None] * sign[None, :]
    return q_lat, q_pe, c_kv, k_pe, w_uv, offsets, L, 1.5 / np.sqrt(r + rope)


@pytest.mark.parametrize("which,aligned", [("queries", False), ("cache", False), ("cache", True)])
def test_error_model_matches_monte_carlo(which, aligned):
    """Pin of attention_error_sigma against the real E4M3 rounding: scaling the
    cache by a (queries by 1 / a) leaves the scores and output / a unchanged
    but moves every value against the E4M3 grid, so the rounding errors of 400
    draws of a in [1, 2) sample the error the model predicts.  Each term alone
    (queries rounded, or the cache rounded) must match within 20 % in total
    variance and within a factor 1.5 element by element (median)."""
    import oracle
    q_lat, q_pe, c_kv, k_pe, w_uv, offsets, L, scale = _mc_problem(aligned)
    B, _, H, r = q_lat.shape
    rows = np.arange(B * L * H)
    exact = oracle.latent_attention(q_lat, q_pe, c_kv, k_pe, w_uv, offsets, L, scale)
    emp = np.zeros_like(exact)
    model = np.zeros_like(exact)
    draws = 400
    for a in 2.0 ** np.random.default_rng(5).uniform(0, 1, draws):
        ql, qp, ck, kp = q_lat / a, q_pe / a, c_kv * a, k_pe * a
        if which == "queries":
            ql, qp = fp8.quantize_query(ql)[0], fp8.quantize_query(qp)[0]
        else:
            codes, sc = fp8.quantize_latent(ck, kp)
            ck, kp = fp8.dequantize_latent(codes, sc, r)
        got = oracle.latent_attention(ql, qp, ck, kp, w_uv, offsets, L, scale) / a
        emp += (got - exact) ** 2
        s = fp8.attention_error_sigma(q_lat / a, q_pe / a, c_kv * a, k_pe * a, w_uv, offsets, L, scale, rows,
                                      queries=which == "queries", cache=which == "cache") / a
        model += s * s
    emp /= draws
    model /= draws
    total = emp.sum() / model.sum()
    per = np.median(emp / model)
    assert 0.8 <= total <= 1.25, f"{which}: empirical / model variance {total:.3f}"
    assert 1 / 1.5 <= per <= 1.5, f"{which}: median element ratio {per:.3f}"


def test_error_model_terms_are_needed():
    """The two terms are of comparable size here, so dropping either one (or the
    value part of the cache term) would fail the Monte Carlo pin above."""
    q_lat, q_pe, c_kv, k_pe, w_uv, offsets, L, scale = _mc_problem()
    rows = np.arange(q_lat.shape[0] * L * q_lat.shape[2])
    sq = fp8.attention_error_sigma(q_lat, q_pe, c_kv, k_pe, w_uv, offsets, L, scale, rows, cache=False)
    sc = fp8.attention_error_sigma(q_lat, q_pe, c_kv, k_pe, w_uv, offsets, L, scale, rows, queries=False)
    both = fp8.attention_error_sigma(q_lat, q_pe, c_kv, k_pe, w_uv, offsets, L, scale, rows)
    ratio = np.sum(sq ** 2) / np.sum(sc ** 2)
    assert 0.2 < ratio < 5, ratio
    assert np.allclose(both ** 2, sq ** 2 + sc ** 2)
