"""GPU parity of the pooled top-k indexer (pooling, scores, selection) with the
oracle, the pages' check that a wide step pools exactly as the same tokens fed
one at a time, the guards on the device path, and the selection feeding the
sparse attention.

Bars: pooled keys within 2^-23 * sum_j |x_j| of the float64 mean (the error
bound of a float32 sum of at most four terms and one division, doubled);
scores within 2^-19 * sum_j |q_j| * mean_rows |x_j| (fourteen float32 roundings
of the dot product, with room for the pooled error); the selection of given
scores bit-exact; the selection of computed scores exact wherever the oracle's
scores separate the budget boundary by more than twice the score bar, and
otherwise valid (nothing left out scores above anything taken, beyond the bar).
"""

import math

import numpy as np
import pytest

from oracle import indexer as ix
from oracle import sparse
from mla_speculative_decode_amd import synth
from tests.helpers import check_close, dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


import mla_speculative_decode_amd as mla  # noqa: E402

U = 2.0 ** -24


def _packed(per_seq):
    keys = np.concatenate(per_seq)
    off = np.concatenate([[0], np.cumsum([len(k) for k in per_seq])]).astype(np.int32)
    return dev(keys, "bf16"), off


def _pool_bar(keys, T):
    """Per window and column: 2^-23 * sum of |x| over the window's rows."""
    a = np.abs(keys[:T].astype(np.float64))
    W = ix.n_windows(T)
    pad = np.zeros((4 * W - T, a.shape[1]))
    return 2.0 * U * np.concatenate([a, pad]).reshape(W, 4, -1).sum(axis=1)


def _score_bar(keys, T, q):
    a = np.abs(keys[:T].astype(np.float64))
    W = ix.n_windows(T)
    cnt = np.minimum(4, T - 4 * np.arange(W))[:, None]
    pad = np.zeros((4 * W - T, a.shape[1]))
    mean_abs = np.concatenate([a, pad]).reshape(W, 4, -1).sum(axis=1) / cnt
    return 2.0 ** -19 * (mean_abs @ np.abs(q.astype(np.float64))) + 1e-30


def _pooled(pool, b, T):
    return pool.pooled[b, :ix.n_windows(T)].double().cpu().numpy()


@pytest.mark.parametrize("d,stride", [(8, 8), (64, 64), (512, 512), (512, 576)])
def test_pool_matches_oracle(d, stride):
    lens = [1, 7, 130]
    x = synth.indexer_inputs(lens, stride, seed=11)
    per = [x.keys[x.offsets[b]:x.offsets[b + 1]] for b in range(3)]
    keys, off = _packed(per)
    pool = mla.IndexerPool(capacity=40, batch_max=4, d=d)
    assert not pool.step(keys, off, S=1)
    torch.cuda.synchronize()
    for b, T in enumerate(lens):
        ref = ix.pool_all(per[b][:, :d], T)
        err = np.abs(_pooled(pool, b, T) - ref)
        assert np.all(err <= _pool_bar(per[b][:, :d], T)), (b, float(err.max()))


@pytest.mark.parametrize("T0", [16, 17, 18, 19])
@pytest.mark.parametrize("S", [2, 3, 4, 8])
def test_wide_step_equals_one_at_a_time(T0, S):
    d = 64
    final = [T0 + S, T0 + 5 + S]
    x = synth.indexer_inputs(final, d, seed=100 + 10 * T0 + S)
    full = [x.keys[x.offsets[b]:x.offsets[b + 1]] for b in range(2)]
    q = torch.from_numpy(x.q).cuda()
    wide = mla.IndexerPool(capacity=16, batch_max=2, d=d)
    narrow = mla.IndexerPool(capacity=16, batch_max=2, d=d)
    start = [T0, T0 + 5]
    keys, off = _packed([full[b][:start[b]] for b in range(2)])
    assert not wide.step(keys, off, S=start[0]) and not narrow.step(keys, off, S=start[0])
    keys, off = _packed(full)
    assert wide.step(keys, off, S=S)
    for k in range(1, S + 1):
        kk, oo = _packed([full[b][:start[b] + k] for b in range(2)])
        assert narrow.step(kk, oo, S=1)
    assert wide.lengths[:2].tolist() == narrow.lengths[:2].tolist() == final
    for b in range(2):
        W = ix.n_windows(final[b])
        assert torch.equal(wide.pooled[b, :W], narrow.pooled[b, :W])
        ref = ix.pool_all(full[b], final[b])
        assert np.all(np.abs(_pooled(wide, b, final[b]) - ref) <= _pool_bar(full[b], final[b]))
    sw = wide.scores(q, off)
    sn = narrow.scores(q, off)
    assert torch.equal(sw, sn)
    for budget in (4, 6, 9):
        a, _ = mla.indexer_select(sw, off, budget)
        c, _ = mla.indexer_select(sn, off, budget)
        assert torch.equal(a, c)


def test_guards_on_the_device_path():
    d = 32
    x = synth.indexer_inputs([40], d, seed=21)
    old = x.keys
    new = np.concatenate([old[:9], synth.draw_like((6, d), 1.0, "bf16", seed=22)])
    pool = mla.IndexerPool(capacity=16, batch_max=2, d=d)
    k18, o18 = _packed([old[:18]])
    assert not pool.step(k18, o18, S=18)
    # cut back to 9 and 2 new tokens, not announced: the length guard forces a full pass
    k11, o11 = _packed([new[:11]])
    assert not pool.plan(o11, S=2)
    assert not pool.step(k11, o11, S=2)
    torch.cuda.synchronize()
    assert np.all(np.abs(_pooled(pool, 0, 11) - ix.pool_all(new, 11)) <= _pool_bar(new, 11))
    # announced trim: the next step stays incremental and exact
    pool.trim([9])
    assert pool.plan(o11, S=2)
    assert pool.step(k11, o11, S=2)
    torch.cuda.synchronize()
    assert np.all(np.abs(_pooled(pool, 0, 11) - ix.pool_all(new, 11)) <= _pool_bar(new, 11))
    # padding or a changed batch shape: full pass
    k15, o15 = _packed([new[:15]])
    assert not pool.step(k15, o15, S=4, padded=True)
    k2, o2 = _packed([new[:15], old[:20]])
    assert not pool.step(k2, o2, S=4)
    torch.cuda.synchronize()
    assert np.all(np.abs(_pooled(pool, 0, 15) - ix.pool_all(new, 15)) <= _pool_bar(new, 15))
    assert np.all(np.abs(_pooled(pool, 1, 20) - ix.pool_all(old, 20)) <= _pool_bar(old, 20))


def _given_scores(W, seed, decimals=1):
    s = synth.draw_like((W,), 1.0, "f32", seed=seed)
    return np.round(s, decimals).astype(np.float32)


def test_select_given_scores_is_exact():
    lens = [1, 5, 6, 10, 2048, 2049, 2051, 700, 9000, 20000]
    budgets = (1, 6, 7, 2048, 5000)   # 5000: positions past the 4096 gathered in LDS are stored directly
    cap = ix.n_windows(max(lens))
    sc = np.zeros((len(lens), cap), dtype=np.float32)
    for b, T in enumerate(lens):
        sc[b, :ix.n_windows(T)] = _given_scores(ix.n_windows(T), seed=30 + b)
    sc[1, :2] = [-0.0, 0.0]
    sc[7, :] = 0.25                                   # all tied
    sc[8, 100:400] = np.float32(1e30)                 # a wide block of equal top scores
    sc[8, 500] = -np.float32(1e30)
    sc[9, :] = 1.5                                    # all tied, more windows than the candidate list holds
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    scd = torch.from_numpy(sc).cuda()
    for budget in budgets:
        sel, soff = mla.indexer_select(scd, off, budget)
        got = sel.cpu().numpy()
        so = soff.host.numpy()
        for b, T in enumerate(lens):
            ref = ix.select_positions(sc[b, :ix.n_windows(T)], T, budget)
            assert np.array_equal(got[so[b]:so[b + 1]], ref), (budget, b, T)


@pytest.mark.parametrize("T", [131072, 140001])
def test_select_large_given_scores_is_exact(T):
    # 131072: every window staged in LDS; 140001: 35001 windows, those past 32768 read from memory
    W = ix.n_windows(T)
    for seed, dec, budget in ((40, 2, 2048), (41, 6, 2048), (42, 3, 9000)):
        s = _given_scores(W, seed, dec)[None, :]
        if T > 131072:
            s[0, -200:] = np.float32(50.0)            # the best windows lie past the staged ones
        sel, _ = mla.indexer_select(torch.from_numpy(s).cuda(), [0, T], budget)
        assert np.array_equal(sel.cpu().numpy(), ix.select_positions(s[0], T, budget)), (seed, budget)


@pytest.mark.parametrize("lens,d", [([37, 1000, 4], 64), ([513], 512), ([77, 300], 520), ([9000], 1024),
                                    # more sequences than the launch has workgroups: one workgroup
                                    # per sequence striding over its groups of windows
                                    ([1 + (37 * i) % 41 for i in range(700)], 64), ([2000] * 600, 8)],
                         ids=["b3", "d512", "d520", "d1024", "b700", "b600_d8"])
def test_scores_match_oracle(lens, d):
    x = synth.indexer_inputs(lens, d, seed=50 + d)
    per = [x.keys[x.offsets[b]:x.offsets[b + 1]] for b in range(len(lens))]
    keys, off = _packed(per)
    pool = mla.IndexerPool(capacity=ix.n_windows(max(lens)), batch_max=len(lens), d=d)
    pool.step(keys, off, S=1)
    got = pool.scores(torch.from_numpy(x.q).cuda(), off).double().cpu().numpy()
    for b, T in enumerate(lens):
        ref = ix.window_scores(ix.pool_all(per[b], T), x.q[b])
        err = np.abs(got[b, :ix.n_windows(T)] - ref)
        assert np.all(err <= _score_bar(per[b], T, x.q[b])), (b, float(err.max()))


def _check_selection(got, ref_scores, T, budget, bar):
    """Count, order, validity against the oracle's scores, and equality with the
    oracle's selection where its boundary is separated by more than 2 * bar."""
    assert got.size == min(budget, T)
    assert np.all(np.diff(got) > 0) and got[0] >= 0 and got[-1] < T
    ref = ix.select_positions(ref_scores, T, budget)
    win = np.arange(T) // 4
    taken = np.zeros(T, dtype=bool)
    taken[got] = True
    if (~taken).any():   # nothing left out beats anything taken by more than the two bars
        assert np.max(ref_scores[win[~taken]] - bar[win[~taken]]) <= np.min(ref_scores[win[taken]] + bar[win[taken]])
    rt = np.zeros(T, dtype=bool)
    rt[ref] = True
    gap = np.min(ref_scores[win[rt]]) - (np.max(ref_scores[win[~rt]]) if (~rt).any() else -np.inf)
    if gap > 2 * bar.max():
        assert np.array_equal(got, ref)


def test_indexer_workload_full_size():
    """The benchmark workload: a pool built over Kv - S positions, one
    incremental step of S, scores and the top-2048 selection; pooled keys
    sampled against the oracle, scores all, the selection validated; the
    incremental pool equals a full recompute bit for bit."""
    wl = synth.INDEXER_WORKLOAD
    T, S, d, budget = wl["kv"], wl["S"], wl["d"], wl["budget"]
    print(f"indexer full size: T={T} S={S} d={d} budget={budget}", flush=True)
    x = synth.indexer_inputs([T], d, seed=wl["seed"])
    keys = dev(x.keys, "bf16")
    cap = ix.n_windows(T)
    inc = mla.IndexerPool(capacity=cap, batch_max=1, d=d)
    assert not inc.step(keys[:T - S], [0, T - S], S=T - S)
    assert inc.step(keys, [0, T], S=S)
    full = mla.IndexerPool(capacity=cap, batch_max=1, d=d)
    assert not full.step(keys, [0, T], S=T)
    torch.cuda.synchronize()
    assert torch.equal(inc.pooled[0], full.pooled[0])
    P = _pooled(inc, 0, T)
    rng = np.random.default_rng(0)
    for w in sorted(set(rng.integers(0, cap, 256).tolist()) | {0, cap - 3, cap - 2, cap - 1}):
        ref = ix.pool_window(x.keys, w, T)
        bar = 2.0 * U * np.abs(x.keys[4 * w:min(4 * w + 4, T)].astype(np.float64)).sum(axis=0)
        assert np.all(np.abs(P[w] - ref) <= bar), w
    q = torch.from_numpy(x.q).cuda()
    got_s = inc.scores(q, [0, T]).double().cpu().numpy()[0]
    ref_s = ix.window_scores(ix.pool_all(x.keys, T), x.q[0])
    sbar = _score_bar(x.keys, T, x.q[0])
    assert np.all(np.abs(got_s - ref_s) <= sbar)
    sel, _ = mla.indexer_select(inc.scores(q, [0, T]), [0, T], budget)
    _check_selection(sel.cpu().numpy(), ref_s, T, budget, sbar)
    # the fused step (tail pooled by the scoring launch) at the same size: same bits
    fused = mla.IndexerPool(capacity=cap, batch_max=1, d=d)
    assert not fused.step(keys[:T - S], [0, T - S], S=T - S)
    sf, was_inc = fused.step_scores(keys, [0, T], S=S, q=q)
    torch.cuda.synchronize()
    assert was_inc
    assert torch.equal(fused.pooled[0], inc.pooled[0])
    assert torch.equal(sf, inc.scores(q, [0, T]))


def test_indexer_feeds_sparse_attention():
    """Pool the latent rows of an MLA cache, score, select, attend: the output
    equals the oracle's attention over the oracle's own selection (the two
    selections are required to agree first)."""
    lens, L, H, r, rope, v, budget = [3000, 1300], 4, 8, 512, 64, 128, 1024
    scale = 1.0 / math.sqrt(128 + rope)
    w_uv = synth.draw_like((H, r, v), 1.0 / math.sqrt(r), "bf16", seed=67)
    c_kv = synth.draw_like((sum(lens), r), 1.0, "bf16", seed=62)
    k_pe = synth.draw_like((sum(lens), rope), 1.0, "bf16", seed=63)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    qi = synth.draw_like((len(lens), r), 1.0 / math.sqrt(r), "f32", seed=64)
    q_lat = synth.draw_like((len(lens), L, H, r), math.sqrt(128 / r), "bf16", seed=65)
    q_pe = synth.draw_like((len(lens), L, H, rope), 1.0, "bf16", seed=66)
    pool = mla.IndexerPool(capacity=ix.n_windows(max(lens)), batch_max=2, d=r)
    pool.step(dev(c_kv, "bf16"), off, S=L)
    scores = pool.scores(torch.from_numpy(qi).cuda(), off)
    sel, soff = mla.indexer_select(scores, off, budget)
    torch.cuda.synchronize()
    got_sel = sel.cpu().numpy()
    ref_sel = []
    for b, T in enumerate(lens):
        keys = c_kv[off[b]:off[b + 1]]
        s = ix.window_scores(ix.pool_all(keys, T), qi[b])
        ref_b = ix.select_positions(s, T, budget)
        assert np.array_equal(got_sel[soff.host[b]:soff.host[b + 1]], ref_b), b
        ref_sel.append(ref_b)
    out = mla.absorbed_attention_sparse(dev(q_lat, "bf16"), dev(q_pe, "bf16"), dev(c_kv, "bf16"),
                                        dev(k_pe, "bf16"), dev(w_uv, "bf16"), off, sel, soff, scale=scale)
    torch.cuda.synchronize()
    ref_soff = np.concatenate([[0], np.cumsum([s.size for s in ref_sel])])
    ref = sparse.sparse_latent_attention(q_lat, q_pe, c_kv, k_pe, w_uv, off, np.concatenate(ref_sel), ref_soff,
                                         L, scale)
    check_close(out.double().cpu().numpy().reshape(-1, v), ref, "bf16", "indexer -> sparse attention")


@pytest.mark.parametrize("d", [64, 520])
def test_step_scores_equals_step_then_scores(d):
    # the fused call pools the tail inside the scoring launch; pooled keys and
    # scores must carry the same bits as the two separate calls, on the full
    # path (first step, padded step) and on the incremental one; a step of 60
    # (at most 16 tail windows: the fused launch, each tail wave taking its
    # groups) and one of 70 (a longer tail: pooled by the pooling kernel first)
    lens0 = [37, 1000, 4, 1]   # the last: every window of the first steps is a tail window
    steps = [(1, False), (3, False), (8, False), (2, True), (5, False), (60, False), (70, False), (4, False)]
    total = [n + sum(s for s, _ in steps) for n in lens0]
    x = synth.indexer_inputs(total, d, seed=90 + d)
    per = [x.keys[x.offsets[b]:x.offsets[b + 1]] for b in range(len(total))]
    cap = ix.n_windows(max(total))
    a = mla.IndexerPool(capacity=cap, batch_max=4, d=d)
    f = mla.IndexerPool(capacity=cap, batch_max=4, d=d)
    qs = synth.draw_like((len(steps) + 1, 4, d), 1.0, "f32", seed=91)
    lens = list(lens0)
    for i, (S, padded) in enumerate([(1, False)] + steps):
        if i > 0:
            lens = [n + S for n in lens]
        keys, off = _packed([p[:n] for p, n in zip(per, lens)])
        q = torch.from_numpy(np.ascontiguousarray(qs[i])).cuda()
        inc_a = a.step(keys, off, S=S, padded=padded)
        sa = a.scores(q, off)
        sf, inc_f = f.step_scores(keys, off, S=S, q=q, padded=padded)
        torch.cuda.synchronize()
        assert inc_a == inc_f, (i, inc_a, inc_f)
        for b, T in enumerate(lens):
            W = ix.n_windows(T)
            assert torch.equal(a.pooled[b, :W], f.pooled[b, :W]), (i, b)
            assert torch.equal(sa[b, :W], sf[b, :W]), (i, b)
    assert inc_f   # the last steps ran the fused tail


def test_fixed_capacity_step_equals_the_ordinary_step():
    # the same steps through step() and step_fixed(): the pooled keys carry the
    # same bits after every step (the fillers write back what they hold); steps
    # that qualify run the fixed shape (capacity 8 or 16), the others (a first
    # step, a step of 20 tokens, a sequence with too few complete windows) the
    # ordinary one
    d = 64
    lens0 = [70, 300, 36]
    steps = [(1, 8), (3, 8), (5, 16), (2, 8), (8, 8), (16, 16), (20, 8), (4, 8), (7, 16)]
    total = [n + sum(s for s, _ in steps) for n in lens0]
    x = synth.indexer_inputs(total, d, seed=131)
    per = [x.keys[x.offsets[b]:x.offsets[b + 1]] for b in range(len(total))]
    cap = ix.n_windows(max(total))
    a = mla.IndexerPool(capacity=cap, batch_max=3, d=d)
    f = mla.IndexerPool(capacity=cap, batch_max=3, d=d)
    lens = list(lens0)
    keys, off = _packed([p[:n] for p, n in zip(per, lens)])
    a.step(keys, off, S=1)            # no pool yet: every window
    inc, c = f.step_fixed(keys, off, S=1)
    assert not inc and c == 0
    seen = set()
    for S, target in steps:
        lens = [n + S for n in lens]
        keys, off = _packed([p[:n] for p, n in zip(per, lens)])
        inc_a = a.step(keys, off, S=S)
        inc_f, c = f.step_fixed(keys, off, S=S, target=target)
        torch.cuda.synchronize()
        assert inc_a and inc_f
        qualifies = S <= 16 and all((n // 4) >= target and ix.n_windows(n) - (n - S) // 4 <= target for n in lens)
        assert c == (target if qualifies else 0), (S, target, lens)
        seen.add(c)
        for b, T in enumerate(lens):
            W = ix.n_windows(T)
            assert torch.equal(a.pooled[b, :W], f.pooled[b, :W]), (S, b)
    assert seen == {0, 8, 16}
    # and against the oracle's pooling of every window
    for b, T in enumerate(lens):
        ref = ix.pool_all(per[b][:T], T)
        got = f.pooled[b, :ix.n_windows(T)].double().cpu().numpy()
        assert np.max(np.abs(got - ref)) <= 1e-5
