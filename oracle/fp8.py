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
