"""Shared helpers for the GPU parity tests: moving seeded inputs to the device
and the comparison bars.

Bars (written here once, used by every parity test):
* float32 storage: max |gpu - oracle| <= 1e-4 (absolute);
* bfloat16 storage, float32 accumulation: |gpu - oracle| <= 2e-2 * scale per
  element, the 2e-2 bar taken relative to the outputs' own scale: the larger of
  the batch rms and the element's row rms (the outputs have rms 0.03-0.4, so
  this is also well inside an absolute 2e-2, which is checked too);
* per element, where a few rows carry much larger outputs than the rest (so that a
  bar relative to the global rms is tighter than the arithmetic allows there):
  the worst-case bound of rounding_bound() below.
"""

from __future__ import annotations

import numpy as np

F32_ABS_TOL = 1e-4
BF16_REL_TOL = 2e-2
# relative error of a score's float32 sum on the matrix cores, as a fraction of
# sum |q_i k_i| (measured 2^-13.6 on the fp8 MFMA with block scales; 4x margin)
MFMA_SUM_REL = 2.0 ** -12


def rounding_bound(q_lat, q_pe, c_kv, k_pe, w_uv, offsets, L: int, scale: float, rows) -> np.ndarray:
    """Worst-case |gpu - exact| per output element of the absorbed path run on
    exactly these values (bf16-exact inputs), from its arithmetic: weights P
    rounded to bf16 (relative 2^-9; the row sums add the same rounded weights),
    score sums off by at most MFMA_SUM_REL sum |q_i k_i| (so P by that times the
    softmax scale), split partial sums stored in bf16 (relative 2^-9), float32
    everywhere else.  A relative change d_t of the weights moves the normalised
    latent output by sum_t w_t d_t (v_t - o) / (1 + sum_t w_t d_t), so with the
    partials
        |do_j| <= sum_t w_t (2^-8 + 2 ds_t) |v_tj - o_j| + 2^-8 sum_t w_t |v_tj|
    (factors of 2 for the second-order terms), and |dout_c| <= sum_j |W_jc| |do_j|
    + 2^-12 sum_j |W_jc o_j| for the float32 up-projection.  rows: flat row ids
    (b L + i) H + h.  Returns [len(rows), v]."""
    q_lat = np.asarray(q_lat, dtype=np.float64)
    B, _, H, r = q_lat.shape
    q_pe = np.zeros((B, L, H, 0)) if q_pe is None else np.asarray(q_pe, dtype=np.float64)
    keys = np.concatenate([np.asarray(c_kv, dtype=np.float64),
                           np.zeros((len(c_kv), 0)) if k_pe is None else np.asarray(k_pe, dtype=np.float64)], axis=1)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    off = np.asarray(offsets, dtype=np.int64)
    out = np.zeros((len(rows), w_uv.shape[2]))
    for n, row in enumerate(rows):
        b, rem = divmod(int(row), L * H)
        i, h = divmod(rem, H)
        vis = int(off[b + 1] - off[b]) - L + i + 1
        K = keys[off[b]:off[b] + vis]
        q = np.concatenate([q_lat[b, i, h], q_pe[b, i, h]])
        s = scale * (K @ q)
        w = np.exp(s - np.max(s))
        w /= np.sum(w)
        V = K[:, :r]
        o = w @ V
        ds = scale * MFMA_SUM_REL * (np.abs(K) @ np.abs(q))
        do = (w * (2.0 ** -8 + 2.0 * ds)) @ np.abs(V - o) + 2.0 ** -8 * (w @ np.abs(V))
        Wa = np.abs(w_uv[h])
        out[n] = do @ Wa + 2.0 ** -12 * (np.abs(o) @ Wa)
    return out


def check_within(got: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str = ""):
    """Element-wise |got - ref| <= bound; returns the largest ratio."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape == bound.shape, (what, got.shape, ref.shape, bound.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ratio = np.abs(got - ref) / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert ratio[worst] <= 1.0, (f"{what}: |err| {abs(got[worst] - ref[worst]):.3e} > bound {bound[worst]:.3e} "
                                 f"at {tuple(int(x) for x in worst)}")
    return float(ratio.max())


def dev(x: np.ndarray, dtype: str, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device).contiguous()


def host64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "", rel: float = BF16_REL_TOL,
                abs_cap: bool = True):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    if dtype == "f32":
        assert err <= F32_ABS_TOL, f"{what}: max abs err {err:.3e} > {F32_ABS_TOL}"
        return err, None
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    # 2e-2 of the output scale: an output row (one attention output, one
    # folded query) is measured against the larger of the batch rms and its
    # own rms, since the bf16 roundings of a row scale with the row (a row led
    # by a few keys has outputs several times the batch rms)
    scale = np.full(ref.shape, max(rms, 1e-30))
    if ref.ndim == 2 and ref.size:
        scale = np.maximum(scale, np.sqrt(np.mean(ref * ref, axis=1))[:, None])
    ratio = np.abs(got - ref) / scale if ref.size else np.zeros(1)
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert ratio[worst] <= rel, (f"{what}: err {float(np.abs(got - ref)[worst]):.3e} > {rel} * scale "
                                 f"{float(scale[worst]):.3e} (batch rms {rms:.3e}) at {tuple(int(x) for x in worst)}")
    if abs_cap:   # outputs of unit-scale inputs: also inside an absolute 2e-2
        assert err <= 2e-2, f"{what}: max err {err:.3e} > 2e-2"
    return err, err / rms


def sample_rows(B: int, L: int, H: int, k: int, seed: int = 0) -> np.ndarray:
    """Row ids (b*L + i)*H + h: every row of a few heads, both ends, and random others."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in {0, B - 1}:
        for i in range(L):
            for h in {0, H - 1}:
                rows.add((b * L + i) * H + h)
    total = B * L * H
    rows.update(int(x) for x in rng.integers(0, total, size=max(0, k - len(rows))))
    return np.array(sorted(rows), dtype=np.int64)
