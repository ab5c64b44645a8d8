"""GPU parity of every C-ABI entry point against the float64 oracle, at sizes
the oracle finishes in seconds that still span several 64-row and 64-position
tiles with ragged tails, variable-length batches, and the degenerate cases
(Kv == L, a single row, a single position)."""

import math

import numpy as np
import pytest

import oracle
from mla_speculative_decode_amd import synth
from tests.helpers import check_close, dev, host64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


import mla_speculative_decode_amd as mla  # noqa: E402

# (name, r, n, v, rope, H, L, kv lengths, dtype)
CASES = [
    ("dsv3_f32_small", 512, 128, 128, 64, 16, 4, [512], "f32"),
    ("f32_ragged_batch", 512, 128, 128, 64, 5, 3, [70, 3, 129], "f32"),
    ("dsv3_bf16_ragged", 512, 128, 128, 64, 24, 5, [300], "bf16"),
    ("dsv3_bf16_batch", 512, 128, 128, 64, 16, 4, [200, 64, 4, 385], "bf16"),
    ("glm47_bf16", 512, 192, 256, 64, 8, 9, [257], "bf16"),
    ("glm53_bf16", 512, 256, 256, 64, 4, 16, [130, 700], "bf16"),
    ("bf16_norope", 512, 128, 128, 0, 8, 8, [190], "bf16"),
    ("bf16_kv_eq_L", 512, 128, 128, 64, 16, 8, [8, 8], "bf16"),
    ("bf16_single_row", 512, 128, 128, 64, 1, 1, [1, 65, 1000], "bf16"),
    # 79 splits of one sequence (merge weights beyond one 64-split window; L = 3 leaves a
    # merge wave without rows)
    ("bf16_many_splits", 512, 128, 128, 64, 2, 3, [5000], "bf16"),
    # L = 20: two merge row tiles of 16, the second ragged
    ("bf16_L20", 512, 128, 128, 64, 4, 20, [100, 333], "bf16"),
    # 130 ragged sequences of 2..200 positions: the split decode and the merge walk the
    # offsets in three chunks of 64 sequences
    ("bf16_batch130", 512, 128, 128, 64, 2, 2, [2 + (37 * i) % 199 for i in range(130)], "bf16"),
]


def _inputs(case, seed=0):
    name, r, n, v, rope, H, L, lens, dt = case
    w = synth.custom(r, n, v, rope, H, len(lens), L, kv=None, kv_range=(1, 1), dtype=dt, seed=seed)
    # explicit lengths: draw with a fixed-length workload per sequence, then pack
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    lens = np.asarray(lens, dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(offs[-1])
    std = 1.0 / math.sqrt(r)
    x = synth.Inputs(w, L, offs,
                     q_nope=synth._draw(rng, (len(lens), L, H, n), 1.0, dt),
                     q_pe=synth._draw(rng, (len(lens), L, H, rope), 1.0, dt),
                     c_kv=synth._draw(rng, (T, r), 1.0, dt),
                     k_pe=synth._draw(rng, (T, rope), 1.0, dt),
                     w_uk=synth._draw(rng, (H, n, r), std, dt),
                     w_uv=synth._draw(rng, (H, r, v), std, dt))
    return x


def _dev_all(x, dt):
    return {k: dev(getattr(x, k), dt) for k in ("q_nope", "q_pe", "c_kv", "k_pe", "w_uk", "w_uv")}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fold_query(case):
    x = _inputs(case)
    dt = case[-1]
    d = _dev_all(x, dt)
    H, n = x.w_uk.shape[0], x.w_uk.shape[1]
    ql = mla.fold_query(d["q_nope"], d["w_uk"])
    torch.cuda.synchronize()
    ref = oracle.fold(x.q_nope.reshape(-1, H, n), x.w_uk).reshape(ql.shape)
    got = host64(ql)
    if dt == "f32":
        check_close(got, ref, dt, "fold")
    else:
        # one bf16 rounding of a float32 sum: within 2^-8 relative, plus accumulation noise
        err = np.abs(got - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5), float(np.max(err - 2.0 ** -8 * np.abs(ref)))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_absorbed_attention_given_q_lat(case):
    x = _inputs(case)
    dt = case[-1]
    name, r, n, v, rope, H, L, lens, _ = case
    # synthetic folded query ~ N(0, n/r), the scale of q_nope . W_UK
    q_lat = synth.draw_like((len(lens), L, H, r), math.sqrt(n / r), dt, seed=77)
    d = _dev_all(x, dt)
    out = mla.absorbed_attention(dev(q_lat, dt), d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"],
                                 x.offsets.astype(np.int32), scale=x.scale)
    torch.cuda.synchronize()
    ref = oracle.latent_attention(q_lat, x.q_pe, x.c_kv, x.k_pe, x.w_uv, x.offsets, L, x.scale)
    check_close(host64(out).reshape(-1, v), ref, dt, f"absorbed_attention {name}")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_absorbed_chain(case):
    # The absorbed route stores the folded query q_lat in the input dtype (bf16): its
    # rounding moves the logits, and rows led by a few keys carry that into outputs
    # several times the batch rms.  As for the materialised chain, the bf16 chain is
    # held to 2e-2 * rms against the oracle that stores its own q_lat in bf16, and to
    # 4e-2 * rms against the exact one.
    x = _inputs(case)
    dt = case[-1]
    name, r, n, v, rope, H, L, lens, _ = case
    d = _dev_all(x, dt)
    out = mla.absorbed(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"],
                       x.offsets.astype(np.int32), scale=x.scale)
    torch.cuda.synchronize()
    ref = oracle.absorbed(x.q_nope, x.q_pe, x.c_kv, x.k_pe, x.w_uk, x.w_uv, x.offsets, x.L, x.scale)
    got = host64(out).reshape(ref.shape)
    if dt == "f32":
        check_close(got, ref, dt, f"absorbed {name}")
        return
    check_close(got, ref, dt, f"absorbed {name} vs exact", rel=4e-2)
    q_lat = oracle.fold(x.q_nope.reshape(-1, H, n), x.w_uk).reshape(len(lens), L, H, r)
    q_lat_q = synth.round_bf16(q_lat.astype(np.float32)).astype(np.float64)
    ref_q = oracle.latent_attention(q_lat_q, x.q_pe, x.c_kv, x.k_pe, x.w_uv, x.offsets, L, x.scale)
    check_close(got, ref_q, dt, f"absorbed {name} vs bf16-stored q_lat")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_materialize_kv(case):
    x = _inputs(case)
    dt = case[-1]
    d = _dev_all(x, dt)
    K, V = mla.materialize_kv(d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"])
    torch.cuda.synchronize()
    Kr, Vr = oracle.expand(x.c_kv, x.k_pe, x.w_uk, x.w_uv)
    gk, gv = host64(K), host64(V)
    if dt == "f32":
        check_close(gk, Kr, dt, "K")
        check_close(gv, Vr, dt, "V")
    else:
        for g, rr, nm in ((gk, Kr, "K"), (gv, Vr, "V")):
            err = np.abs(g - rr)
            assert np.all(err <= 2.0 ** -8 * np.abs(rr) + 1e-4), nm
        # the rope part is a copy: exact
        n = x.w_uk.shape[1]
        assert np.array_equal(gk[:, :, n:], Kr[:, :, n:])


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_materialized_attention_given_kv(case):
    x = _inputs(case)
    dt = case[-1]
    name, r, n, v, rope, H, L, lens, _ = case
    if dt == "bf16" and not (n in (128, 192, 256) and rope in (0, 64) and v in (128, 256)):
        pytest.skip("geometry not compiled for bf16 materialised attention")
    T = int(x.offsets[-1])
    K = synth.draw_like((T, H, n + rope), 1.0, dt, seed=31)
    V = synth.draw_like((T, H, v), 1.0, dt, seed=32)
    d = _dev_all(x, dt)
    out = mla.materialized_attention(d["q_nope"], d["q_pe"], dev(K, dt), dev(V, dt),
                                     x.offsets.astype(np.int32), scale=x.scale)
    torch.cuda.synchronize()
    ref = oracle.attention(x.q_nope, x.q_pe, K, V, x.offsets, L, x.scale, n=n)
    check_close(host64(out).reshape(ref.shape), ref, dt, f"materialized_attention {name}")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_materialized_chain(case):
    # The materialised route stores the expanded K and V in the input dtype
    # (bf16): that storage rounding alone moves outputs by about 2.6e-2 * rms at
    # these sizes (float64 simulation of the oracle with K, V rounded to bf16).
    # So the chain is held to 2e-2 * rms against the oracle that applies the same
    # storage rounding to its own K and V, and to 4e-2 * rms against the exact one.
    x = _inputs(case)
    dt = case[-1]
    name, r, n, v, rope, H, L, lens, _ = case
    if dt == "bf16" and not (n in (128, 192, 256) and rope in (0, 64) and v in (128, 256)):
        pytest.skip("geometry not compiled for bf16 materialised attention")
    d = _dev_all(x, dt)
    out = mla.materialized(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"],
                           x.offsets.astype(np.int32), scale=x.scale)
    torch.cuda.synchronize()
    got = host64(out).reshape(-1, v)
    ref = oracle.materialized(x.q_nope, x.q_pe, x.c_kv, x.k_pe, x.w_uk, x.w_uv, x.offsets, x.L, x.scale)
    if dt == "f32":
        check_close(got, ref, dt, f"materialized {name}")
        return
    check_close(got, ref, dt, f"materialized {name} vs exact", rel=4e-2)
    K, V = oracle.expand(x.c_kv, x.k_pe, x.w_uk, x.w_uv)
    Kq = synth.round_bf16(K.astype(np.float32)).astype(np.float64)
    Vq = synth.round_bf16(V.astype(np.float32)).astype(np.float64)
    ref_q = oracle.attention(x.q_nope, x.q_pe, Kq, Vq, x.offsets, L, x.scale, n=n)
    check_close(got, ref_q, dt, f"materialized {name} vs bf16-stored K/V")


def test_two_gpu_paths_agree():
    case = CASES[2]
    x = _inputs(case)
    d = _dev_all(x, "bf16")
    offs = x.offsets.astype(np.int32)
    a = mla.absorbed(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"], offs, scale=x.scale)
    m = mla.materialized(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"], offs, scale=x.scale)
    torch.cuda.synchronize()
    ref = oracle.absorbed(x.q_nope, x.q_pe, x.c_kv, x.k_pe, x.w_uk, x.w_uv, x.offsets, x.L, x.scale)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert float(torch.max(torch.abs(a - m))) <= 4e-2 * rms


def test_deterministic():
    case = CASES[3]
    x = _inputs(case)
    d = _dev_all(x, "bf16")
    offs = mla.Offsets(x.offsets.astype(np.int32))
    outs = [mla.absorbed(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"], offs, scale=x.scale)
            for _ in range(3)]
    mats = [mla.materialized(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"], offs,
                             scale=x.scale) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    assert torch.equal(mats[0], mats[1])


def test_select_path_through_binding():
    g = mla.Geom(512, 192, 256, 64, 32)
    assert mla.select_path(g, 379, 8192) == (mla.MLA_ABSORBED, 379)
    assert mla.select_path(g, 380, 8192) == (mla.MLA_MATERIALIZED, 379)
    assert mla.select_path(g, 398, 0) == (mla.MLA_ABSORBED, 398)



def _ramp(T: int, kind: str) -> np.ndarray:
    """Per-position factors on the keys that spread the logits of a row over a
    wide range: a sawtooth of period 256 positions rising from 1 to 81 (within
    each period the last tiles exceed the first by far more than 2^64), the
    falling sawtooth, and one late key scaled by 80."""
    t = (np.arange(T) % 256) / 255.0
    if kind == "rising":
        f = 1.0 + 80.0 * t
    elif kind == "falling":
        f = 81.0 - 80.0 * t
    else:
        f = np.ones(T)
        f[(T * 7) // 8] = 80.0
    return f.astype(np.float32)


@pytest.mark.parametrize("kind", ["rising", "falling", "spike"])
def test_wide_score_range(kind):
    """Logits of one row spread over hundreds of log2 units (keys scaled by
    position) on both attention kernels.  At these shapes the plans cut the
    4096 positions into splits of 256 (absorbed: 16 row tiles of 64; materialised:
    16 heads x 1 row tile), so every split holds one rise of the sawtooth: the
    fixed per-row reference of the kernels must be raised inside a split."""
    r, n, v, rope, L, kv = 512, 128, 128, 64, 8, 4096
    H = 128
    x = _inputs(("wide", r, n, v, rope, H, L, [kv], "bf16"))
    f = _ramp(kv, kind)
    c_kv = synth.round_bf16(x.c_kv * f[:, None])
    k_pe = synth.round_bf16(x.k_pe * f[:, None])
    q_lat = synth.draw_like((1, L, H, r), math.sqrt(n / r), "bf16", seed=78)
    offs = x.offsets.astype(np.int32)
    if kind == "rising":
        # precondition: in some split of 256 positions a row's later tile exceeds its
        # first tile's maximum by more than 64 (log2 units)
        s = (q_lat.reshape(-1, r).astype(np.float64) @ c_kv[:512].astype(np.float64).T
             + x.q_pe.reshape(-1, rope).astype(np.float64) @ k_pe[:512].astype(np.float64).T) * x.scale / math.log(2)
        assert np.max(s[:, 192:256].max(1) - s[:, 0:64].max(1)) > 64
    d = _dev_all(x, "bf16")
    out = mla.absorbed_attention(dev(q_lat, "bf16"), d["q_pe"], dev(c_kv, "bf16"), dev(k_pe, "bf16"), d["w_uv"],
                                 offs, scale=x.scale)
    torch.cuda.synchronize()
    ref = oracle.latent_attention(q_lat, x.q_pe, c_kv, k_pe, x.w_uv, x.offsets, L, x.scale)
    # keys scaled up to 81x give outputs of rms up to ~50: the bar is relative only
    check_close(host64(out).reshape(-1, v), ref, "bf16", f"absorbed_attention {kind}", abs_cap=False)

    Hm = 16
    xm = _inputs(("wide_m", r, n, v, rope, Hm, L, [kv], "bf16"))
    K = synth.round_bf16(synth.draw_like((kv, Hm, n + rope), 1.0, "bf16", seed=33) * f[:, None, None])
    V = synth.draw_like((kv, Hm, v), 1.0, "bf16", seed=34)
    dm = _dev_all(xm, "bf16")
    outm = mla.materialized_attention(dm["q_nope"], dm["q_pe"], dev(K, "bf16"), dev(V, "bf16"), offs, scale=xm.scale)
    torch.cuda.synchronize()
    refm = oracle.attention(xm.q_nope, xm.q_pe, K, V, xm.offsets, L, xm.scale, n=n)
    check_close(host64(outm).reshape(refm.shape), refm, "bf16", f"materialized_attention {kind}", abs_cap=False)
