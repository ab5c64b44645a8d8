"""Shared helpers for the GPU parity tests: moving seeded inputs to the device
and the comparison bars.

Bars (written here once, used by every parity test):
* float32 storage: max |gpu - oracle| <= 1e-4 (absolute);
* bfloat16 storage, float32 accumulation: max |gpu - oracle| <= 2e-2 * rms(oracle)
  (the 2e-2 bar taken relative to the outputs' own scale; these outputs have
  rms 0.03-0.1, so this is also well inside an absolute 2e-2).
"""

from __future__ import annotations

import numpy as np

F32_ABS_TOL = 1e-4
BF16_REL_TOL = 2e-2


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
    assert err <= rel * max(rms, 1e-30), f"{what}: max err {err:.3e} > {rel} * rms {rms:.3e}"
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
