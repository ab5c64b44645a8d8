"""GPU parity of the absorbed attention over selected positions
(mla_absorbed_attention_sparse) against the float64 oracle, and bit-identity
with the dense path when every position is selected."""

import math

import numpy as np
import pytest

from oracle import sparse
from mla_speculative_decode_amd import synth
from tests.helpers import check_close, dev, host64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


import mla_speculative_decode_amd as mla  # noqa: E402
from tests.test_parity_gpu import _inputs  # noqa: E402


def _sel_dev(sels):
    sel = np.concatenate(sels).astype(np.int32)
    soff = np.concatenate([[0], np.cumsum([s.size for s in sels])]).astype(np.int32)
    return sel, soff, torch.from_numpy(sel).cuda()


def _run(case, sels, seed=77):
    name, r, n, v, rope, H, L, lens, dt = case
    x = _inputs(case)
    q_lat = synth.draw_like((len(lens), L, H, r), math.sqrt(n / r), dt, seed=seed)
    sel, soff, sel_d = _sel_dev(sels)
    out = mla.absorbed_attention_sparse(dev(q_lat, dt), dev(x.q_pe, dt) if rope else None, dev(x.c_kv, dt),
                                        dev(x.k_pe, dt) if rope else None, dev(x.w_uv, dt),
                                        x.offsets.astype(np.int32), sel_d, soff, scale=x.scale)
    torch.cuda.synchronize()
    ref = sparse.sparse_latent_attention(q_lat, x.q_pe, x.c_kv, x.k_pe, x.w_uv, x.offsets, sel, soff, L, x.scale)
    return x, q_lat, out, ref


def test_full_selection_equals_dense_path():
    case = ("full", 512, 128, 128, 64, 16, 4, [300, 77], "bf16")
    name, r, n, v, rope, H, L, lens, dt = case
    x, q_lat, out, ref = _run(case, [np.arange(k) for k in lens])
    dense = mla.absorbed_attention(dev(q_lat, dt), dev(x.q_pe, dt), dev(x.c_kv, dt), dev(x.k_pe, dt),
                                   dev(x.w_uv, dt), x.offsets.astype(np.int32), scale=x.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, dense)
    check_close(host64(out).reshape(-1, v), ref, "bf16", "sparse full selection")


@pytest.mark.parametrize("case,budgets", [
    (("dsv3_sel", 512, 128, 128, 64, 8, 8, [3000, 700], "bf16"), (512, 300)),
    (("glm53_sel", 512, 256, 256, 64, 4, 16, [4000], "bf16"), (2048,)),
    (("norope_sel", 512, 128, 128, 0, 8, 4, [1000, 90, 400], "bf16"), (100, 90, 257)),
])
def test_random_selections(case, budgets):
    name, r, n, v, rope, H, L, lens, dt = case
    rng = np.random.default_rng(len(name))
    sels = []
    for k, m in zip(lens, budgets):
        s = rng.choice(k - 4, size=m - 4, replace=False)
        s = np.concatenate([s, np.arange(k - 4, k)])     # the newest positions are selected too
        sels.append(np.sort(s))
    x, q_lat, out, ref = _run(case, sels)
    check_close(host64(out).reshape(-1, v), ref, "bf16", f"sparse {name}")
    # deterministic: a second call (fresh workspace) gives the same bits
    sel, soff, sel_d = _sel_dev(sels)
    again = mla.absorbed_attention_sparse(dev(q_lat, dt), dev(x.q_pe, dt) if rope else None, dev(x.c_kv, dt),
                                          dev(x.k_pe, dt) if rope else None, dev(x.w_uv, dt),
                                          x.offsets.astype(np.int32), sel_d, soff, scale=x.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, again)


def test_rows_that_see_nothing_output_zero():
    case = ("late_sel", 512, 128, 128, 64, 4, 8, [200], "bf16")
    name, r, n, v, rope, H, L, lens, dt = case
    x, q_lat, out, ref = _run(case, [np.array([195, 197, 199])])
    got = host64(out).reshape(L, H, v)
    assert np.all(got[:3] == 0)       # row i sees positions < 193 + i: rows 0..2 see none of 195, 197, 199
    assert np.all(np.any(got[3:] != 0, axis=-1))
    check_close(got.reshape(-1, v), ref, "bf16", "sparse late selection")


def test_long_block_counts_visible_entries_by_search():
    # L = 80 rows: a row's invisible entries are among the selection's last
    # L - 1 = 79 > 64, so the kernel counts each row's visible entries by a
    # binary search of the selection instead of from one register of its tail
    case = ("long_block", 512, 128, 128, 64, 2, 80, [600, 300], "bf16")
    name, r, n, v, rope, H, L, lens, dt = case
    rng = np.random.default_rng(66)
    sels = []
    for k in lens:
        old = rng.choice(k - L, size=90, replace=False)             # positions every row sees
        new = rng.choice(np.arange(k - L, k), size=50, replace=False)   # among the block's own rows
        sels.append(np.sort(np.concatenate([old, new, [k - 1]])))
    x, q_lat, out, ref = _run(case, [np.unique(s) for s in sels])
    check_close(host64(out).reshape(-1, v), ref, "bf16", "sparse long block")


def test_positions_past_2_22_are_addressed():
    # A cache of 2^22 + 192 positions (4.3 GB of latent rows): the latent and
    # rope rows of selected positions past 2^22 lie beyond what a 32-bit
    # element offset (position x 512) reaches.  The dense and selected-position
    # kernels share the row-address code, so this covers both.  Only the
    # selected rows hold data; the oracle runs on those rows packed densely, with
    # the block's own rows kept last, which leaves every row's view unchanged
    # (a row i sees position p iff p < Kv - L + i + 1).
    r, rope, H, L, v = 512, 64, 2, 4, 128
    Kv = (1 << 22) + 192
    rng = np.random.default_rng(22)
    old = np.sort(np.concatenate([rng.choice(1000, 20, replace=False),
                                  (1 << 22) - 64 + rng.choice(64, 8, replace=False),
                                  (1 << 22) + rng.choice(Kv - L - (1 << 22), 30, replace=False)]))
    sel = np.concatenate([np.unique(old), np.arange(Kv - L, Kv)]).astype(np.int32)
    k = sel.size
    rows = synth.draw_like((k, r), 1.0, "bf16", seed=221)
    ropes = synth.draw_like((k, rope), 1.0, "bf16", seed=222)
    q_lat = synth.draw_like((1, L, H, r), math.sqrt(128 / r), "bf16", seed=223)
    q_pe = synth.draw_like((1, L, H, rope), 1.0, "bf16", seed=224)
    w_uv = synth.draw_like((H, r, v), 1.0 / math.sqrt(r), "bf16", seed=225)
    scale = 1.0 / math.sqrt(128 + rope)
    c_kv = torch.zeros((Kv, r), dtype=torch.bfloat16, device="cuda")
    k_pe = torch.zeros((Kv, rope), dtype=torch.bfloat16, device="cuda")
    idx = torch.from_numpy(sel.astype(np.int64)).cuda()
    c_kv[idx] = dev(rows, "bf16")
    k_pe[idx] = dev(ropes, "bf16")
    soff = np.array([0, k], dtype=np.int32)
    out = mla.absorbed_attention_sparse(dev(q_lat, "bf16"), dev(q_pe, "bf16"), c_kv, k_pe, dev(w_uv, "bf16"),
                                        np.array([0, Kv], dtype=np.int32), torch.from_numpy(sel).cuda(), soff,
                                        scale=scale)
    torch.cuda.synchronize()
    del c_kv, k_pe
    m = k - L   # packed: the old selected rows first, then the block's own L rows
    ref = sparse.sparse_latent_attention(q_lat, q_pe, rows, ropes, w_uv, np.array([0, k]), np.arange(k), soff,
                                         L, scale)
    assert m == int(np.sum(sel < Kv - L))
    check_close(host64(out).reshape(-1, v), ref, "bf16", "sparse past 2^22")
