"""Pins of the selected-position (sparse) attention oracle: the full selection
reproduces the dense oracle (an independent C implementation), a one-row block
equals dense attention over the gathered cache, a single visible position gives
its value row through W_UV, and rows that see nothing output zero."""

import math

import numpy as np

import oracle
from oracle import sparse


def _inp(B=2, L=4, H=3, r=32, rope=8, v=16, lens=(40, 23), seed=0):
    rng = np.random.default_rng(seed)
    offs = np.concatenate([[0], np.cumsum(lens)])
    T = int(offs[-1])
    return dict(q_lat=rng.standard_normal((B, L, H, r)), q_pe=rng.standard_normal((B, L, H, rope)),
                c_kv=rng.standard_normal((T, r)), k_pe=rng.standard_normal((T, rope)),
                w_uv=rng.standard_normal((H, r, v)) / math.sqrt(r), offsets=offs, L=L,
                scale=1 / math.sqrt(24))


def test_full_selection_is_dense():
    d = _inp()
    lens = np.diff(d["offsets"])
    sel = np.concatenate([np.arange(k) for k in lens])
    soff = d["offsets"]
    got = sparse.sparse_latent_attention(d["q_lat"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"], d["offsets"],
                                         sel, soff, d["L"], d["scale"])
    ref = oracle.latent_attention(d["q_lat"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"], d["offsets"], d["L"],
                                  d["scale"])
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_one_row_equals_dense_over_gathered_cache():
    d = _inp(L=1, lens=(50, 31))
    rng = np.random.default_rng(3)
    sels = [np.sort(rng.choice(k, size=m, replace=False)) for k, m in zip(np.diff(d["offsets"]), (17, 9))]
    sel = np.concatenate(sels)
    soff = np.concatenate([[0], np.cumsum([s.size for s in sels])])
    got = sparse.sparse_latent_attention(d["q_lat"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"], d["offsets"],
                                         sel, soff, 1, d["scale"])
    rows = np.concatenate([d["offsets"][b] + s for b, s in enumerate(sels)])
    ref = oracle.latent_attention(d["q_lat"], d["q_pe"], d["c_kv"][rows], d["k_pe"][rows], d["w_uv"], soff, 1,
                                  d["scale"])
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_single_visible_position_and_empty_rows():
    d = _inp(B=1, L=4, lens=(30,))
    sel = np.array([5, 28])            # 28 is visible to rows i >= 2 only (28 < 30 - 4 + i + 1)
    got = sparse.sparse_latent_attention(d["q_lat"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"], d["offsets"],
                                         sel, np.array([0, 2]), 4, d["scale"]).reshape(4, 3, -1)
    want = np.einsum("c,hcv->hv", d["c_kv"][5], d["w_uv"])
    assert np.allclose(got[0], want, atol=1e-12) and np.allclose(got[1], want, atol=1e-12)
    sel2 = np.array([27, 29])          # row 0 sees positions < 27: nothing
    got2 = sparse.sparse_latent_attention(d["q_lat"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"], d["offsets"],
                                          sel2, np.array([0, 2]), 4, d["scale"]).reshape(4, 3, -1)
    assert np.all(got2[0] == 0) and np.allclose(got2[1], np.einsum("c,hcv->hv", d["c_kv"][27], d["w_uv"]),
                                                atol=1e-12)
