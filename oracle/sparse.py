"""Absorbed attention over selected cache positions.

TEST INFRASTRUCTURE ONLY (the oracle): imported by the tests, the smoke check
and the benchmark's CPU-baseline leg, never by the product path.

"One guard, 110x off the verify step", section "The sparse model is
different": an indexer selects the top 2048 cached positions and attention
runs only over those.  Readings: the selection is per sequence (shared by the
verify block's L rows and all heads), given as positions from the sequence
start; row i attends to the selected positions it may see under the dense
causal rule (p < Kv - L + i + 1); a row that sees none of them outputs zero.
Written as plain loops over (sequence, row) in float64.
"""

from __future__ import annotations

import numpy as np


def sparse_latent_attention(q_lat, q_pe, c_kv, k_pe, w_uv, offsets, sel, sel_offsets, L, scale):
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_pe = np.asarray(k_pe, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    B, _, H, r = q_lat.shape
    v = w_uv.shape[-1]
    out = np.zeros((B, L, H, v))
    for b in range(B):
        o0, kv = int(offsets[b]), int(offsets[b + 1] - offsets[b])
        chosen = np.asarray(sel[int(sel_offsets[b]):int(sel_offsets[b + 1])], dtype=np.int64)
        for i in range(L):
            vis = chosen[chosen < kv - L + i + 1]
            if vis.size == 0:
                continue
            ck = c_kv[o0 + vis]                                   # [n, r]
            kp = k_pe[o0 + vis]                                   # [n, rope]
            s = (q_lat[b, i] @ ck.T + q_pe[b, i] @ kp.T) * scale   # [H, n]
            s -= s.max(axis=1, keepdims=True)
            w = np.exp(s)
            w /= w.sum(axis=1, keepdims=True)
            o_lat = w @ ck                                        # [H, r]
            out[b, i] = np.einsum("hc,hcv->hv", o_lat, w_uv)
    return out.reshape(B * L * H, v)
