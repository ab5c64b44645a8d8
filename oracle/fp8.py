"""fp8 (OCP E4M3) latent cache: encoding, per-position scaling, dequantisation.

TEST INFRASTRUCTURE ONLY (the oracle): imported by the tests, the smoke check
and the benchmark's CPU-baseline leg, never by the product path.

The pages test a "quantised latent form" of the cache without defining it
(mlx-lm PR #1817, section "Tests"); this is the reading built here:
* element format: OCP 8-bit floating point E4M3 -- 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent 0 holds the subnormals m x 2^-9;
  no infinities; S.1111.111 is NaN, so the largest finite value is
  1.75 x 2^8 = 448;
* one scale per cached position, shared by its latent and rope parts: the
  smallest power of two 2^k with max|x| <= 448 x 2^k (k in [-126, 127];
  k = 0 for an all-zero row), so that x / 2^k is exact in float32 and the
  dequantised values code x 2^k are exact in bfloat16;
* encoding rounds to the nearest E4M3 value, ties to the even code, and
  saturates at 448 (the scale keeps every |x| / 2^k <= 448, so it never has to);
* the attention of the fp8 path is the attention over the dequantised cache.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode(codes) -> np.ndarray:
    """E4M3 code (uint8) -> value (float64; NaN for 0x7f / 0xff)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return s * val


# every finite non-negative E4M3 value, in code order (codes 0x00 .. 0x7e)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = decode(_POS_CODES)


def encode(y) -> np.ndarray:
    """Finite values -> E4M3 codes: nearest value, ties to the even code,
    magnitudes above 448 saturate to 448.  Written as a search over the 127
    non-negative values (no bit tricks), so it is checked against decode()."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    # index of the largest value <= a, and the next one up
    lo = np.searchsorted(_POS_VALUES, a, side="right") - 1
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, hi, lo)
    sign = (y < 0) & (code != 0)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def row_scale_exponent(amax) -> np.ndarray:
    """Smallest k with amax <= 448 x 2^k, clamped to [-126, 127]; 0 for amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    k = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    # 448 x 2^k >= amax  <=>  k >= log2(amax / 448); evaluated exactly by stepping
    kk = np.ceil(np.log2(np.where(nz, amax, 1.0) / E4M3_MAX)).astype(np.int64)
    kk = np.where(E4M3_MAX * np.exp2(kk.astype(np.float64) - 1) >= amax, kk - 1, kk)   # guard a log2 rounding
    kk = np.where(E4M3_MAX * np.exp2(kk.astype(np.float64)) < amax, kk + 1, kk)
    k = np.where(nz, kk, 0)
    return np.clip(k, -126, 127)


def quantize_latent(c_kv, k_pe):
    """Rows [c_kv[t] | k_pe[t]] -> (codes uint8 [T, r + rope], scales float32 [T] = 2^k)."""
    x = np.concatenate([np.asarray(c_kv, dtype=np.float64), np.asarray(k_pe, dtype=np.float64)], axis=1)
    k = row_scale_exponent(np.max(np.abs(x), axis=1))
    codes = encode(x * np.exp2(-k.astype(np.float64))[:, None])
    return codes, np.exp2(k.astype(np.float64)).astype(np.float32)


def dequantize_latent(codes, scales, r: int):
    """(codes, scales) -> (c_kv_hat [T, r], k_pe_hat [T, rope]) in float64 (exact)."""
    x = decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]
    return x[:, :r], x[:, r:]


# ---- block-quantised queries ----------------------------------------------------
# The fp8 path also rounds the queries to E4M3 so that the scores run on fp8
# matrix hardware.  The pages fix nothing about it; the reading built here: one
# power-of-two scale per block of 32 consecutive values of a query row (q_lat and
# q_pe blocked separately), chosen by the same rule as a cache row's.

QUERY_BLOCK = 32


def quantize_query(q, block: int = QUERY_BLOCK):
    """Query rows (last axis, a multiple of `block`) -> (dequantised values
    float64, codes uint8, exponents k per block): codes = encode(q / 2^k) with
    2^k the smallest power of two holding the block's max|q| <= 448 x 2^k."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    if d == 0:
        return q.copy(), np.zeros(q.shape, dtype=np.uint8), np.zeros(q.shape[:-1] + (0,), dtype=np.int64)
    assert d % block == 0, "query width must be a multiple of the block"
    blocks = q.reshape(q.shape[:-1] + (d // block, block))
    k = row_scale_exponent(np.max(np.abs(blocks), axis=-1))
    codes = encode(blocks * np.exp2(-k.astype(np.float64))[..., None])
    deq = decode(codes) * np.exp2(k.astype(np.float64))[..., None]
    return deq.reshape(q.shape), codes.reshape(q.shape), k


# ---- error model: E4M3 rounding of queries and cache, against exact inputs ----------
# First order in the rounding errors, each taken as an independent variable
# spread evenly over one E4M3 step of its value (variance step^2 / 12).  For one
# query row with exact scores s_t = scale (q . k_t), weights w = softmax(s) over
# the visible positions, up-projected values u_t = c_t W (W = that head's
# W_UV) and output o = sum_t w_t u_t, a change ds_t of the scores and dc_t of
# the value rows moves the output by
#     do = sum_t w_t (ds_t (u_t - o) + dc_t W).
# Query errors e (shared by every position) give ds_t = scale (e . k_t); cache
# errors n_t give ds_t = scale (q . n_t) and dc_t = the latent part of n_t.  So
#     var(o_c) = sum_i var(e_i) G_ic^2,   G = scale K^T (w (u - o))        (queries)
#              + sum_t w_t^2 sum_j var(n_tj) (scale q_j (u_tc - o_c) + [j < r] W_jc)^2   (cache)


def e4m3_rounding_variance(x, k):
    """Variance of the error of rounding x / 2^k to E4M3 (then x 2^k): one step of
    the grid at |x| / 2^k (2^(e - 3) in the binade [2^e, 2^(e+1)), 2^-9 below
    2^-6), squared, times 4^k, over 12.  Zero for x == 0."""
    x = np.asarray(x, dtype=np.float64)
    kk = np.asarray(k, dtype=np.float64)
    y = np.abs(x) * np.exp2(-kk)
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    step = np.exp2(e - 3.0 + kk)
    return np.where(y == 0, 0.0, step * step / 12.0)


def attention_error_sigma(q_lat, q_pe, c_kv, k_pe, w_uv, offsets, L: int, scale: float, rows,
                          queries: bool = True, cache: bool = True):
    """Standard deviation, per output element, of the absorbed attention's error
    when the queries (blocks of 32) and/or the cache rows are rounded to E4M3 as
    above.  rows: flat query-row ids (b L + i) H + h.  Returns [len(rows), v]."""
    q_lat = np.asarray(q_lat, dtype=np.float64)
    B, Lq, H, r = q_lat.shape
    assert Lq == L
    q_pe = np.zeros((B, L, H, 0)) if q_pe is None else np.asarray(q_pe, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_pe = np.zeros((c_kv.shape[0], 0)) if k_pe is None else np.asarray(k_pe, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    off = np.asarray(offsets, dtype=np.int64)
    keys = np.concatenate([c_kv, k_pe], axis=1)
    if cache:
        kc = row_scale_exponent(np.max(np.abs(keys), axis=1))
        var_n = e4m3_rounding_variance(keys, kc[:, None])
    out = np.zeros((len(rows), w_uv.shape[2]))
    for n, row in enumerate(rows):
        b, rem = divmod(int(row), L * H)
        i, h = divmod(rem, H)
        T = int(off[b + 1] - off[b])
        vis = T - L + i + 1
        K = keys[off[b]:off[b] + vis]
        q = np.concatenate([q_lat[b, i, h], q_pe[b, i, h]])
        s = scale * (K @ q)
        w = np.exp(s - np.max(s))
        w /= np.sum(w)
        W = w_uv[h]                                   # [r, v]
        U = K[:, :r] @ W                              # [vis, v]
        o = w @ U
        D = U - o
        var = np.zeros(W.shape[1])
        if queries:
            qs = [quantize_query(q_lat[b, i, h])[2]]
            if q_pe.shape[-1]:
                qs.append(quantize_query(q_pe[b, i, h])[2])
            kq = np.concatenate([np.repeat(x, QUERY_BLOCK) for x in qs])
            var_e = e4m3_rounding_variance(q, kq)
            G = scale * (K.T @ (w[:, None] * D))      # [r + rope, v]
            var += var_e @ (G * G)
        if cache:
            vn = var_n[off[b]:off[b] + vis]
            A = vn @ (q * q)                          # [vis]
            Bm = (vn[:, :r] * q[None, :r]) @ W        # [vis, v]
            C = vn[:, :r] @ (W * W)                   # [vis, v]
            w2 = (w * w)[:, None]
            var += np.sum(w2 * (scale * scale * D * D * A[:, None] + 2.0 * scale * D * Bm + C), axis=0)
        out[n] = np.sqrt(var)
    return out
