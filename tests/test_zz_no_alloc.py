"""The entry point that allocates nothing (mla_absorbed_attention_noalloc),
through the C ABI: two calls in a row on one GPU, the second on a smaller
input, each against mla_absorbed_attention on the same inputs (the same
kernels and plan, so the same bits), and the second call checked after the
first left the shared scratch array full of its own partials."""

import math

import numpy as np
import pytest

from mla_speculative_decode_amd import synth
from tests.helpers import dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


import mla_speculative_decode_amd as mla  # noqa: E402


def _case(H, L, lens, dt, seed):
    r, n, v, rope = 512, 128, 128, 64
    B = len(lens)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(offs[-1])
    x = {"q_lat": synth.draw_like((B, L, H, r), math.sqrt(n / r), dt, seed=seed),
         "q_pe": synth.draw_like((B, L, H, rope), 1.0, dt, seed=seed + 1),
         "c_kv": synth.draw_like((T, r), 1.0, dt, seed=seed + 2),
         "k_pe": synth.draw_like((T, rope), 1.0, dt, seed=seed + 3),
         "w_uv": synth.draw_like((H, r, v), 1.0 / math.sqrt(r), dt, seed=seed + 4)}
    d = {k: dev(a, dt) for k, a in x.items()}
    return d, mla.Offsets(offs, "cuda"), 1.0 / math.sqrt(n + rope), (B, L, H, v)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_matches_the_workspace_call(dt):
    # first call: the 128-head, 8-row verify step over 8192 positions (bf16), then a
    # smaller one (two sequences, fewer heads and rows): its partials overwrite
    # only part of what the first call left in the array
    cases = [(128, 8, [8192], 11), (16, 4, [700, 77], 21)] if dt == "bf16" else [(16, 4, [512], 31),
                                                                                 (4, 2, [90, 33], 41)]
    for H, L, lens, seed in cases:
        d, offs, scale, shape = _case(H, L, lens, dt, seed)
        out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        mla.absorbed_attention_noalloc(d["q_lat"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"], offs, out, scale,
                                       n=128)
        ref = mla.absorbed_attention(d["q_lat"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"], offs, scale=scale)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), (H, L, lens)
        assert torch.equal(out, ref), (H, L, lens, float((out - ref).abs().max()))
