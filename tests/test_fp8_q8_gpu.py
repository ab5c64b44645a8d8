"""GPU parity of the fp8 route with the queries quantised once, by the fold
(mla_fold_query_fp8 and mla_absorbed_attention_fp8q):

* the fold's q_lat equals mla_fold_query's, bit for bit;
* the E4M3 query block, read back through the layout the attention kernel
  uses, equals the oracle's block quantisation (oracle fp8.quantize_query) of
  those bf16 rows and of q_pe: codes and scale exponents bit for bit, with
  all-zero rows, widely scaled rows and the encoding's corner cases (ties,
  448 x 2^k, subnormals) in the rope part.  One representational freedom: a
  negative value that rounds to zero may carry its sign (code 0x80, the
  hardware conversion's) where the oracle writes 0x00; both are the value 0,
  so codes are compared with the sign of zero cleared;
* the attention over that block equals mla_absorbed_attention_fp8, which
  quantises q_lat and q_pe inside its kernel, bit for bit."""

import numpy as np
import pytest

from oracle import fp8
from mla_speculative_decode_amd import synth
from tests.helpers import dev, host64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


import mla_speculative_decode_amd as mla  # noqa: E402
from tests.test_fp8_gpu import _edge_rows  # noqa: E402

TILE, ROPE_OFF, SCALE_OFF = 19456, 16384, 18432

# (name, H, L, sequence lengths, rope, n, v)
CASES = [
    ("h16_l3_b2_ragged_tile", 16, 3, [700, 800], 64, 128, 128),
    ("h128_l8_b1", 128, 8, [2048], 64, 128, 128),
    ("h16_l4_rope0", 16, 4, [1500], 0, 128, 128),
    ("h32_l8_n192_v256", 32, 8, [3000], 64, 192, 256),
    ("h64_l16_b3", 64, 16, [600, 2100, 50], 64, 256, 256),
]


def decode_q8(q8: np.ndarray, B: int, L: int, H: int, rope: int):
    """The query block -> (codes [B, L H, 512 + rope] uint8, exponents [B, L H,
    16 + rope / 32]): row l H + h of sequence b in tile (l H + h) / 32; lane
    16 (k % 64 / 16) + row % 16 of fragment (row / 16, k / 128), half k % 128 /
    64, byte k % 16; the rope step's lane groups hold its 64 values; one scale
    byte (e + 127) per 32-wide block, in its lane group."""
    t = q8.reshape(B, -1, TILE)
    rows = np.arange(L * H)
    rt, rr = rows // 32, rows % 32
    k = np.arange(512)
    f = (rr[:, None] >> 4) * 4 + k[None, :] // 128
    half = (k[None, :] % 128) // 64
    lane = 16 * ((k[None, :] % 64) // 16) + rr[:, None] % 16
    codes = [t[:, rt[:, None], 16 * ((2 * f + half) * 64 + lane) + k[None, :] % 16]]
    jj = np.arange(16)
    exps = [t[:, rt[:, None], SCALE_OFF + 4 * (128 * (rr[:, None] >> 4) + 16 * (jj[None, :] % 4) + rr[:, None] % 16)
              + jj[None, :] // 4].astype(np.int64) - 127]
    if rope:
        kr = np.arange(rope)
        codes.append(t[:, rt[:, None], ROPE_OFF + 16 * (64 * (rr[:, None] >> 4) + 16 * (kr[None, :] // 16)
                                                        + rr[:, None] % 16) + kr[None, :] % 16])
        j = np.arange(rope // 32)
        exps.append(t[:, rt[:, None], SCALE_OFF + 4 * (64 * (2 * (rr[:, None] >> 4) + 1) + 16 * j[None, :]
                                                       + rr[:, None] % 16)].astype(np.int64) - 127)
    return np.concatenate(codes, axis=-1), np.concatenate(exps, axis=-1)


def _inputs(case, seed):
    name, H, L, lens, rope, n, v = case
    B = len(lens)
    rng = np.random.default_rng(seed)
    # rows of widely different magnitude, some all zero
    q_nope = rng.standard_normal((B, L, H, n)) * np.exp(rng.uniform(-8, 8, (B, L, H, 1)))
    q_nope[0, 0, : min(H, 3)] = 0.0
    q_pe = rng.standard_normal((B, L, H, rope)) * np.exp(rng.uniform(-8, 8, (B, L, H, 1)))
    if rope:
        _, ek = _edge_rows(512, rope)
        m = min(len(ek), H)
        q_pe[-1, -1, :m] = ek[:m]
    w_uk = rng.standard_normal((H, n, 512)) / np.sqrt(n)
    T = int(sum(lens))
    c_kv = rng.standard_normal((T, 512))
    k_pe = rng.standard_normal((T, rope))
    w_uv = rng.standard_normal((H, 512, v)) / np.sqrt(512)
    r32 = lambda a: synth.round_bf16(a.astype(np.float32))
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return [r32(a) for a in (q_nope, q_pe, w_uk, c_kv, k_pe, w_uv)] + [offs]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fold_q8_codes_and_attention(case):
    name, H, L, lens, rope, n, v = case
    B = len(lens)
    q_nope, q_pe, w_uk, c_kv, k_pe, w_uv, offs = _inputs(case, 11)
    print(f"case {name}", flush=True)
    dq, dw = dev(q_nope, "bf16"), dev(w_uk, "bf16")
    dpe = dev(q_pe, "bf16") if rope else None
    q_lat = mla.fold_query(dq, dw)
    q_lat8, q8 = mla.fold_query_fp8(dq, dw, dpe, q_lat=True)
    torch.cuda.synchronize()
    assert torch.equal(q_lat.view(torch.int16), q_lat8.view(torch.int16)), "fold_query_fp8's q_lat differs from fold_query's"

    # the query block against the oracle's quantisation of the same bf16 rows
    ql = host64(q_lat).reshape(B, L * H, 512)
    qfull = np.concatenate([ql, q_pe.astype(np.float64).reshape(B, L * H, rope)], axis=-1) if rope else ql
    _, want_codes, want_k = fp8.quantize_query(qfull)
    got_codes, got_k = decode_q8(q8.cpu().numpy(), B, L, H, rope)
    got_codes = np.where((got_codes & 0x7F) == 0, 0, got_codes)   # -0 and +0: the same value
    bad = np.argwhere(got_codes != want_codes)
    assert bad.size == 0, f"{len(bad)} query codes differ, first at {bad[:3].tolist()}"
    assert np.array_equal(got_k, want_k), "query block scales differ"

    # the attention over the block equals the in-kernel quantisation's, bit for bit
    codes, scales = mla.quantize_latent_fp8(dev(c_kv, "bf16"), dev(k_pe, "bf16") if rope else None)
    dwuv = dev(w_uv, "bf16")
    scale = 1.0 / np.sqrt(n + rope)
    a = mla.absorbed_attention_fp8(q_lat, dpe, codes, scales, dwuv, offs, scale=scale)
    b = mla.absorbed_attention_fp8q(q8, B, L, codes, scales, dwuv, offs, scale, rope=rope)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32)), \
        f"max |diff| {float((a - b).abs().max())}"
