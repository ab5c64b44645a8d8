"""Pins of the float64 oracle against facts fixed outside itself (CPU only).

* two-path identity: the absorbed and materialised routes are mathematically
  equivalent ("One guard, 110x off the verify step", section "The defect"), so
  the oracle's two independent implementations must agree to float64 rounding;
* reduction to a library routine: with selection matrices as W_UK / W_UV, MLA
  is ordinary multi-head attention over gathered latent columns, which
  torch.nn.functional.scaled_dot_product_attention computes (float64, CPU);
* closed forms: a single visible key, uniform attention, the causal cut;
* invariants: a constant logit shift, a permutation of visible keys.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from mla_speculative_decode_amd import synth


def _inp(r=64, n=32, v=48, rope=16, H=3, B=2, L=4, kv=(9, 17), seed=0):
    rng = np.random.default_rng(seed)
    lens = np.asarray(kv, dtype=np.int64)
    assert lens.size == B
    offs = np.concatenate([[0], np.cumsum(lens)])
    T = int(offs[-1])
    d = dict(
        q_nope=rng.standard_normal((B, L, H, n)),
        q_pe=rng.standard_normal((B, L, H, rope)),
        c_kv=rng.standard_normal((T, r)),
        k_pe=rng.standard_normal((T, rope)),
        w_uk=rng.standard_normal((H, n, r)) / math.sqrt(r),
        w_uv=rng.standard_normal((H, r, v)) / math.sqrt(r),
        offsets=offs, L=L, scale=1.0 / math.sqrt(n + rope))
    return d


def _abs(d, **kw):
    return oracle.absorbed(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"],
                           d["offsets"], d["L"], d["scale"], **kw)


def _mat(d):
    return oracle.materialized(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"],
                               d["offsets"], d["L"], d["scale"])


@pytest.mark.parametrize("shape", [
    dict(),
    dict(r=32, n=32, v=32, rope=0, H=2, B=1, L=1, kv=(1,)),
    dict(r=96, n=64, v=16, rope=8, H=4, B=3, L=5, kv=(5, 6, 40)),
    dict(r=128, n=16, v=128, rope=32, H=1, B=1, L=8, kv=(64,)),
])
def test_two_paths_agree(shape):
    d = _inp(**shape)
    a, m = _abs(d), _mat(d)
    assert a.shape == m.shape
    assert np.max(np.abs(a - m)) <= 1e-12 * max(1.0, np.max(np.abs(m)))


def test_composition_of_halves():
    d = _inp()
    H, L = d["w_uk"].shape[0], d["L"]
    ql = oracle.fold(d["q_nope"].reshape(-1, H, d["q_nope"].shape[-1]), d["w_uk"])
    a2 = oracle.latent_attention(ql, d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"], d["offsets"], L, d["scale"])
    assert np.array_equal(a2, _abs(d))
    K, V = oracle.expand(d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"])
    m2 = oracle.attention(d["q_nope"], d["q_pe"], K, V, d["offsets"], L, d["scale"], n=d["q_nope"].shape[-1])
    assert np.max(np.abs(m2 - _mat(d))) <= 1e-13
    # selected rows and positions equal the full computation
    sel = np.array([0, 5, 7, 13, 2 * L * H - 1])
    assert np.array_equal(_abs(d, sel=sel), _abs(d)[sel])
    tsel = np.array([3, 0, 25])
    K2, V2 = oracle.expand(d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"], tsel=tsel)
    assert np.array_equal(K2, K[tsel]) and np.array_equal(V2, V[tsel])


def _sdpa_reference(q, k, v, L, offsets, scale):
    """torch SDPA (float64, CPU) per sequence with an explicit boolean causal mask.
    q [B, L, H, dq], k [T, H, dq], v [T, H, dv] -> [B, L, H, dv]."""
    outs = []
    for b in range(len(offsets) - 1):
        o0, o1 = int(offsets[b]), int(offsets[b + 1])
        Kv = o1 - o0
        qb = torch.from_numpy(q[b]).permute(1, 0, 2)          # [H, L, dq]
        kb = torch.from_numpy(k[o0:o1]).permute(1, 0, 2)      # [H, Kv, dq]
        vb = torch.from_numpy(v[o0:o1]).permute(1, 0, 2)
        i = torch.arange(L)[:, None]
        t = torch.arange(Kv)[None, :]
        mask = t < (Kv - L + i + 1)
        ob = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask, scale=scale)
        outs.append(ob.permute(1, 0, 2).numpy())
    return np.stack(outs)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_selection_weights_reduce_to_mha(seed):
    # W_UK[h, j, c] = [c == pi_h(j)], W_UV[h, c, e] = [c == sigma_h(e)]: then
    # K_h = [c_kv[:, pi_h] | k_pe], V_h = c_kv[:, sigma_h], Q_h = [q_nope_h | q_pe_h].
    # A transposed or mis-indexed weight picks different columns and fails.
    r, n, v, rope, H, B, L = 40, 12, 9, 6, 3, 2, 3
    d = _inp(r=r, n=n, v=v, rope=rope, H=H, B=B, L=L, kv=(7, 11), seed=seed)
    rng = np.random.default_rng(100 + seed)
    pis = [rng.permutation(r)[:n] for _ in range(H)]
    sigmas = [rng.permutation(r)[:v] for _ in range(H)]
    w_uk = np.zeros((H, n, r)); w_uv = np.zeros((H, r, v))
    for h in range(H):
        w_uk[h, np.arange(n), pis[h]] = 1.0
        w_uv[h, sigmas[h], np.arange(v)] = 1.0
    d["w_uk"], d["w_uv"] = w_uk, w_uv
    k = np.stack([np.concatenate([d["c_kv"][:, pis[h]], d["k_pe"]], axis=1) for h in range(H)], axis=1)
    vv = np.stack([d["c_kv"][:, sigmas[h]] for h in range(H)], axis=1)
    q = np.concatenate([d["q_nope"], d["q_pe"]], axis=-1)
    ref = _sdpa_reference(q, k, vv, L, d["offsets"], d["scale"]).reshape(-1, v)
    for got in (_abs(d), _mat(d)):
        assert np.max(np.abs(got - ref)) <= 1e-12


def test_identity_weights_reduce_to_mqa():
    # n = v = r and identity weights: MQA with K = [c_kv | k_pe], V = c_kv shared by heads.
    r, rope, H, B, L = 24, 8, 4, 1, 5
    d = _inp(r=r, n=r, v=r, rope=rope, H=H, B=B, L=L, kv=(13,), seed=7)
    d["w_uk"] = np.stack([np.eye(r)] * H)
    d["w_uv"] = np.stack([np.eye(r)] * H)
    k = np.repeat(np.concatenate([d["c_kv"], d["k_pe"]], axis=1)[:, None, :], H, axis=1)
    vv = np.repeat(d["c_kv"][:, None, :], H, axis=1)
    q = np.concatenate([d["q_nope"], d["q_pe"]], axis=-1)
    ref = _sdpa_reference(q, k, vv, L, d["offsets"], d["scale"]).reshape(-1, r)
    assert np.max(np.abs(_abs(d) - ref)) <= 1e-12
    assert np.max(np.abs(_mat(d) - ref)) <= 1e-12


def test_single_visible_key():
    # Kv = L = 1: softmax over one key is 1, so out = c_kv[0] @ W_UV[h].
    d = _inp(B=1, L=1, kv=(1,))
    H = d["w_uk"].shape[0]
    ref = np.stack([d["c_kv"][0] @ d["w_uv"][h] for h in range(H)])
    assert np.max(np.abs(_abs(d) - ref)) <= 1e-13
    assert np.max(np.abs(_mat(d) - ref)) <= 1e-13


def test_zero_query_is_uniform_mean():
    # q = 0: every visible key has weight 1/vis, so out = mean(c_kv[:vis]) @ W_UV[h].
    d = _inp(B=2, L=4, kv=(6, 10))
    d["q_nope"][:] = 0.0
    d["q_pe"][:] = 0.0
    H, L = d["w_uk"].shape[0], d["L"]
    out = _abs(d).reshape(2, L, H, -1)
    mout = _mat(d).reshape(2, L, H, -1)
    for b in range(2):
        o0 = d["offsets"][b]
        Kv = d["offsets"][b + 1] - o0
        for i in range(L):
            vis = Kv - L + i + 1
            mean = d["c_kv"][o0:o0 + vis].mean(axis=0)
            for h in range(H):
                ref = mean @ d["w_uv"][h]
                assert np.max(np.abs(out[b, i, h] - ref)) <= 1e-13
                assert np.max(np.abs(mout[b, i, h] - ref)) <= 1e-13


def test_causal_cut():
    # Row i sees positions < Kv - L + i + 1: changing position Kv - L + i + 1 leaves
    # rows <= i unchanged and changes row i + 1.
    d = _inp(B=1, L=4, kv=(12,))
    H, L, Kv = d["w_uk"].shape[0], d["L"], 12
    base = _abs(d).reshape(L, H, -1)
    for i in range(L - 1):
        t = Kv - L + i + 1
        d2 = {k: (x.copy() if isinstance(x, np.ndarray) else x) for k, x in d.items()}
        d2["c_kv"][t] += 3.0
        d2["k_pe"][t] -= 2.0
        got = _abs(d2).reshape(L, H, -1)
        assert np.array_equal(got[: i + 1], base[: i + 1])
        assert np.max(np.abs(got[i + 1] - base[i + 1])) > 1e-6
        gm = _mat(d2).reshape(L, H, -1)
        assert np.max(np.abs(gm[: i + 1] - base[: i + 1])) <= 1e-12


def test_constant_logit_shift_invariance():
    # An extra rope coordinate that is constant over keys adds the same amount to
    # every logit of a row: the softmax, hence the output, is unchanged.
    d = _inp(seed=3)
    ref = _abs(d)
    rng = np.random.default_rng(9)
    d2 = dict(d)
    d2["q_pe"] = np.concatenate([d["q_pe"], rng.standard_normal(d["q_pe"].shape[:-1] + (1,)) * 5], axis=-1)
    d2["k_pe"] = np.concatenate([d["k_pe"], np.full((d["k_pe"].shape[0], 1), 2.5)], axis=-1)
    assert np.max(np.abs(_abs(d2) - ref)) <= 1e-12
    assert np.max(np.abs(_mat(d2) - ref)) <= 1e-12


def test_visible_key_permutation_invariance():
    # Positions every row sees (the first Kv - L + 1) may be permuted freely.
    d = _inp(B=1, L=3, kv=(15,), seed=4)
    ref = _abs(d)
    perm = np.random.default_rng(5).permutation(15 - 3 + 1)
    d2 = dict(d)
    c = d["c_kv"].copy(); k = d["k_pe"].copy()
    c[: perm.size] = d["c_kv"][perm]; k[: perm.size] = d["k_pe"][perm]
    d2["c_kv"], d2["k_pe"] = c, k
    assert np.max(np.abs(_abs(d2) - ref)) <= 1e-13


def test_scale_is_applied_to_both_terms():
    # Doubling scale equals doubling both q_nope and q_pe (logits are bilinear).
    d = _inp(seed=6)
    d2 = dict(d)
    d2["scale"] = 2 * d["scale"]
    d3 = dict(d)
    d3["q_nope"] = 2 * d["q_nope"]; d3["q_pe"] = 2 * d["q_pe"]
    assert np.max(np.abs(_abs(d2) - _abs(d3))) <= 1e-13


def test_synthetic_inputs_are_storage_exact():
    w = synth.custom(64, 32, 32, 16, 2, 2, 3, kv_range=(3, 9), dtype="bf16", seed=11)
    x = synth.make_inputs(w)
    for a in (x.q_nope, x.q_pe, x.c_kv, x.k_pe, x.w_uk, x.w_uv):
        assert a.dtype == np.float32
        assert np.array_equal(synth.round_bf16(a), a)
        t = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(t, a)
    # numpy rounding matches torch's round-to-nearest-even on arbitrary floats
    y = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    assert np.array_equal(synth.round_bf16(y), torch.from_numpy(y).to(torch.bfloat16).float().numpy())
    assert np.all(np.diff(x.offsets) >= 3) and x.offsets[0] == 0
    # reproducible
    assert np.array_equal(synth.make_inputs(w).c_kv, x.c_kv)
