"""GPU parity of every stage against the CPU oracle, at sizes the oracle
finishes in seconds that still span several tiles and a ragged tail, plus the
edge cases: ragged and empty requests, every token a candidate, all-equal
scores, negative weights, padded selections, empty row lists.

Integer stages (compact keys, candidates, top-k positions and scores, slot
resolution, gathered bytes) must match bit for bit; attention within 2e-2
(bf16 output) and 1e-4 (fp32 log-sum-exp)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from top_sparse_attention_ls_amd import synth
from tests.gpu_common import (OUT_TOL, LSE_TOL, np_, bits, bf16_to_f64, oracle_cand,
                              oracle_topk, poison_, assert_attention_close)

pytestmark = pytest.mark.gpu
DEV = "cuda"

TINY = synth.WORKLOADS["tiny-4k"]
SHRUNK = dataclasses.replace(synth.WORKLOADS["decode-128k-b32"], name="shrunk-128k", batch=3,
                             ctx=8192 + 37, n_cand=1024, topk=256, planted=82, hot_slots=512)


def idx_inputs(wl, ctx_len=None, device="cpu"):
    return synth.indexer_inputs(wl, device, ctx_len=ctx_len)


# ------------------------------------------------------------------ pack --

@pytest.mark.parametrize("D", [64, 128])
def test_pack_coarse_bit_exact(ls, D):
    g = torch.Generator().manual_seed(D)
    k = torch.randint(-128, 128, (777, D), generator=g, dtype=torch.int32).to(torch.int8)
    k[0, :] = torch.arange(-128, 128, dtype=torch.int32)[:D].to(torch.int8)
    k[1, :] = torch.arange(-128, 128, dtype=torch.int32)[-D:].to(torch.int8)
    got = np_(ls.pack_coarse(k.to(DEV)))
    assert np.array_equal(got, orc.pack_coarse(k.numpy()))


# -------------------------------------------------- coarse + candidates --

def run_coarse_case(ls, inp, ctx_len, C):
    q, w, keys = inp["q"], inp["w"], inp["keys"]
    kc = ls.pack_coarse(keys.to(DEV))
    cl = torch.tensor(ctx_len, dtype=torch.int32, device=DEV)
    cand = ls.index_coarse(q.to(DEV), w.to(DEV), kc, cl, C)
    got = np_(cand)
    for b in range(q.shape[0]):
        exp = oracle_cand(q[b].numpy(), w[b].numpy(), keys[b].numpy(), ctx_len[b], C)
        assert got[b].tolist() == exp.tolist(), "request %d" % b
    return got


def test_index_coarse_tiny(ls):
    inp = idx_inputs(TINY)
    got = run_coarse_case(ls, inp, [TINY.ctx], TINY.n_cand)
    # planted tokens are strong: all of them are candidates
    planted = set(inp["planted"][0].tolist())
    assert planted <= set(got[0].tolist())


def test_index_coarse_shrunk_ragged(ls):
    ctx = [SHRUNK.ctx, 5000, 700]            # full (ragged tail), partial, fewer than C
    inp = idx_inputs(SHRUNK, ctx_len=ctx)
    run_coarse_case(ls, inp, ctx, SHRUNK.n_cand)


def test_index_coarse_empty_and_tiny_requests(ls):
    wl = dataclasses.replace(SHRUNK, batch=4, ctx=3000)
    ctx = [0, 1, 63, 3000]
    inp = idx_inputs(wl, ctx_len=ctx)
    got = run_coarse_case(ls, inp, ctx, 1024)
    assert got[0].tolist() == [-1] * 1024
    assert got[1].tolist() == [0] + [-1] * 1023


def test_index_coarse_all_equal_scores(ls):
    # every key identical: every score ties, the lowest positions win
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=20000)
    inp = idx_inputs(wl)
    inp["keys"][:] = inp["keys"][:, :1, :]
    got = run_coarse_case(ls, inp, [20000, 20000], 1024)
    assert got[0].tolist() == list(range(1024))


def test_index_coarse_few_distinct_scores(ls):
    # keys drawn from 3 patterns: huge tie groups cross the threshold
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=12000)
    inp = idx_inputs(wl)
    g = torch.Generator().manual_seed(3)
    pick = torch.randint(0, 3, (2, 12000), generator=g)
    for b in range(2):
        inp["keys"][b] = inp["keys"][b, :3][pick[b]]
    run_coarse_case(ls, inp, [12000, 11111], 1000)


def test_index_coarse_negative_weights(ls):
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=9000)
    inp = idx_inputs(wl)
    g = torch.Generator().manual_seed(4)
    inp["w"] = torch.randint(-128, 128, inp["w"].shape, generator=g, dtype=torch.int32).to(torch.int8)
    run_coarse_case(ls, inp, [9000, 8999], 777)


# up to 16 heads one 16-head tile, more heads 32-head tiles (one or two)
@pytest.mark.parametrize("H,D", [(4, 64), (16, 128), (17, 128), (20, 64), (32, 128), (33, 128),
                                 (64, 64)])
def test_index_coarse_head_shapes(ls, H, D):
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=6000, idx_heads=H, idx_dim=D)
    inp = idx_inputs(wl)
    run_coarse_case(ls, inp, [6000, 4321], 500)


def test_index_coarse_balanced_grid(ls):
    # 64 requests of 40000 tokens fill fewer than 512 workgroups at 8192
    # tokens each, so the launch cuts every row into 8 pieces of 5120 tokens
    # (workgroup boundaries off the 8192 grid); ragged lengths end mid-piece
    wl = dataclasses.replace(SHRUNK, batch=64, ctx=40000, idx_heads=4, idx_dim=64)
    ctx = [40000 - 613 * b for b in range(64)]
    inp = idx_inputs(wl, ctx_len=ctx)
    run_coarse_case(ls, inp, ctx, 700)


def test_index_coarse_every_token_a_candidate(ls):
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=3000)
    inp = idx_inputs(wl)
    got = run_coarse_case(ls, inp, [3000, 2000], 4096)
    assert got[0].tolist()[:3000] == list(range(3000))


# ------------------------------------------------------ refine + top-k --

def run_refine_case(ls, inp, ctx_len, C, K, k8=None, kpos2slot=None, kcache=None):
    """k8: the key store the library reads (default: the keys, on the
    device); the oracle always scores with the true keys inp["keys"]."""
    q, w, keys = inp["q"], inp["w"], inp["keys"]
    B = q.shape[0]
    cands = np.stack([oracle_cand(q[b].numpy(), w[b].numpy(), keys[b].numpy(), ctx_len[b], C)
                      for b in range(B)])
    cl = torch.tensor(ctx_len, dtype=torch.int32, device=DEV)
    tk, sc = ls.refine_topk(q.to(DEV), w.to(DEV), keys.to(DEV) if k8 is None else k8,
                            torch.from_numpy(cands).to(DEV), cl, K, kpos2slot=kpos2slot,
                            kcache=kcache)
    tk, sc = np_(tk), np_(sc)
    for b in range(B):
        ep, es = oracle_topk(q[b].numpy(), w[b].numpy(), keys[b].numpy(), cands[b], K)
        assert tk[b].tolist() == ep.tolist(), "request %d positions" % b
        assert sc[b].tolist() == es.tolist(), "request %d scores" % b
    return tk


def test_refine_topk_tiny(ls):
    inp = idx_inputs(TINY)
    tk = run_refine_case(ls, inp, [TINY.ctx], TINY.n_cand, TINY.topk)
    assert set(inp["planted"][0].tolist()) <= set(tk[0].tolist())


def test_refine_topk_shrunk_ragged(ls):
    ctx = [SHRUNK.ctx, 3000, 200]
    inp = idx_inputs(SHRUNK, ctx_len=ctx)
    run_refine_case(ls, inp, ctx, SHRUNK.n_cand, SHRUNK.topk)


def test_refine_topk_k_above_candidates(ls):
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=5000)
    inp = idx_inputs(wl)
    run_refine_case(ls, inp, [5000, 100], 300, 400)


def test_refine_topk_ties(ls):
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=6000)
    inp = idx_inputs(wl)
    g = torch.Generator().manual_seed(5)
    pick = torch.randint(0, 4, (2, 6000), generator=g)
    for b in range(2):
        inp["keys"][b] = inp["keys"][b, :4][pick[b]]
    run_refine_case(ls, inp, [6000, 6000], 2000, 333)


def test_refine_topk_more_than_16384_candidates(ls):
    # C > 16384: the per-request block selection (k_topk) instead of the
    # histogram slices; a ragged second request with fewer valid tokens
    # than C
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=40000)
    ctx = [40000, 17000]
    inp = idx_inputs(wl, ctx_len=ctx)
    run_refine_case(ls, inp, ctx, 20000, 2048)


def test_refine_topk_tie_list_overflow(ls):
    # more than 8192 candidates in the threshold bucket: the histogram
    # kernel's tie list cannot hold them and the exact cut runs over every
    # candidate in global memory.  Request 0: every key equal (all 10000
    # candidates tie, the lowest 333 positions win).  Request 1: 100 strong
    # tokens, 9500 of one equal weaker score with the cut inside that group,
    # weak tokens after
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=12000)
    inp = idx_inputs(wl)
    q, w, keys = inp["q"], inp["w"], inp["keys"]
    keys[0] = keys[0, :1]
    pats = ordered_patterns(q[1].numpy(), w[1].numpy(), keys[1])
    g = torch.Generator().manual_seed(12)
    perm = torch.randperm(12000, generator=g)
    lvl = torch.full((12000,), 2, dtype=torch.long)
    lvl[perm[:100]] = 0
    lvl[perm[100:9600]] = 1
    keys[1] = pats[lvl]
    tk = run_refine_case(ls, inp, [12000, 12000], 10000, 333)
    assert tk[0].tolist() == list(range(333))


def wide_bucket_of(x):
    """The float-like bucket of an int64 score (exact below 128, then 64 per
    power of two): used only to build two different scores that share a
    bucket."""
    x = int(x)

    def mag(y):
        if y < 128:
            return y
        e = y.bit_length() - 1
        return 128 + (e - 7) * 64 + ((y >> (e - 6)) & 63)
    return mag(x) if x >= 0 else -1 - mag(-(x + 1))


def near_pattern(q, w, row):
    """A copy of key row `row` with one element moved by one whose fine score
    differs from the row's but lies in the same bucket."""
    base = int(orc.index_scores(q, w, row[None].numpy(), False)[0])
    for d in range(row.shape[0]):
        for delta in (1, -1):
            v = int(row[d]) + delta
            if not -128 <= v <= 127:
                continue
            r = row.clone()
            r[d] = v
            sc = int(orc.index_scores(q, w, r[None].numpy(), False)[0])
            if sc != base and wide_bucket_of(sc) == wide_bucket_of(base):
                return r
    raise AssertionError("no near pattern")


def test_refine_topk_long_tie_lists(ls):
    # more than 2048 ties in the threshold bucket, all within the LDS list.
    # Request 0: 3000 tokens of one equal score with the cut inside the group
    # (the one-key shortcut, ties ranked by position).  Request 1: the same
    # 3000 tokens split between two different scores of one bucket, the cut
    # inside the lower one (the shortcut must not apply; the workgroup search
    # runs).  Every token is a candidate, 200 strong ones above the group.
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=6000)
    inp = idx_inputs(wl)
    q, w, keys = inp["q"], inp["w"], inp["keys"]
    g = torch.Generator().manual_seed(21)
    for b in range(2):
        pats = ordered_patterns(q[b].numpy(), w[b].numpy(), keys[b])
        perm = torch.randperm(6000, generator=g)
        lvl = torch.full((6000,), 2, dtype=torch.long)
        lvl[perm[:200]] = 0
        lvl[perm[200:3200]] = 1
        rows = pats[lvl]
        if b == 1:
            rows[perm[1700:3200]] = near_pattern(q[b].numpy(), w[b].numpy(), pats[1])
        keys[b] = rows
    run_refine_case(ls, inp, [6000, 6000], 6000, 2400)


def test_refine_topk_pinned_host_keys(ls):
    # the original keys stay in pinned host memory; the refinement reads the
    # candidates' rows over PCIe
    ctx = [SHRUNK.ctx, 3000, 200]
    inp = idx_inputs(SHRUNK, ctx_len=ctx)
    run_refine_case(ls, inp, ctx, SHRUNK.n_cand, SHRUNK.topk, k8=inp["keys"].pin_memory())


def cached_key_store(wl, inp, ctx, C, rate, S, host):
    """Key cache holding (1 - rate) of the oracle's candidates; the k8 rows of
    cached tokens are overwritten with unrelated keys (so a read of k8 for a
    cached token changes the result), and a few uncached tokens get slot
    values outside [0, S), which must count as absent."""
    q, w, keys = inp["q"], inp["w"], inp["keys"]
    B = q.shape[0]
    cands = torch.stack([torch.from_numpy(oracle_cand(q[b].numpy(), w[b].numpy(),
                                                      keys[b].numpy(), ctx[b], C))
                         for b in range(B)])
    kp, kcache, n_miss = synth.key_cache_fill(wl, cands, keys, "cpu", miss_rate=rate,
                                              key_slots=S)
    store = keys.clone()
    g = torch.Generator().manual_seed(23)
    cached = kp >= 0
    junk = torch.randint(-127, 128, (int(cached.sum()), keys.shape[2]), generator=g,
                         dtype=torch.int32).to(torch.int8)
    store[cached] = junk
    for b in range(B):
        miss = [int(t) for t in cands[b] if t >= 0 and kp[b, int(t)] < 0][:8]
        for i, t in enumerate(miss):
            kp[b, t] = S + i if i % 2 == 0 else -2 - i
    assert (sum(n_miss) > 0) == (rate > 0)
    return (store.pin_memory() if host else store.to(DEV)), kp.to(DEV), kcache.to(DEV)


@pytest.mark.parametrize("host", [True, False], ids=["host-keys", "device-keys"])
def test_refine_topk_key_cache(ls, host):
    ctx = [SHRUNK.ctx, 3000, 200]
    inp = idx_inputs(SHRUNK, ctx_len=ctx)
    k8, kp, kcache = cached_key_store(SHRUNK, inp, ctx, SHRUNK.n_cand, 0.3, 1500, host)
    run_refine_case(ls, inp, ctx, SHRUNK.n_cand, SHRUNK.topk, k8=k8, kpos2slot=kp,
                    kcache=kcache)


def test_refine_topk_key_cache_d64_all_cached(ls):
    # head_dim 64, every candidate cached: k8 is never read for a candidate
    wl = dataclasses.replace(TINY, batch=2, ctx=3000)
    ctx = [3000, 1700]
    inp = idx_inputs(wl, ctx_len=ctx)
    k8, kp, kcache = cached_key_store(wl, inp, ctx, 1024, 0.0, 1024, True)
    run_refine_case(ls, inp, ctx, 1024, 256, k8=k8, kpos2slot=kp, kcache=kcache)


def ordered_patterns(q, w, keys):
    """Three key rows whose coarse and fine scores both strictly decrease."""
    cs = orc.index_scores(q, w, keys[:256].numpy(), True)
    fs = orc.index_scores(q, w, keys[:256].numpy(), False)
    order = np.lexsort((-cs, -fs))
    for i in range(1, len(order) - 1):
        hi, mid = order[0], order[i]
        if not (fs[hi] > fs[mid] and cs[hi] > cs[mid]):
            continue
        for lo in order[::-1]:
            if fs[mid] > fs[lo] and cs[mid] > cs[lo]:
                return keys[[int(hi), int(mid), int(lo)]].clone()
    raise AssertionError("no ordered patterns")


def three_level_patterns(q, w, keys, coarse):
    """Three key rows of strictly decreasing (coarse or fine) score."""
    s = orc.index_scores(q, w, keys[:64].numpy(), coarse)
    order = np.argsort(-s, kind="stable")
    hi, mid, lo = order[0], order[len(order) // 2], order[-1]
    assert s[hi] > s[mid] > s[lo]
    return keys[[int(hi), int(mid), int(lo)]].clone()


@pytest.mark.parametrize("stage", ["coarse", "fine"])
def test_cut_inside_a_short_equal_group(ls, stage):
    # strong tokens, then 50 tokens of one equal score with the cut inside
    # that group (its 20 lowest positions win), then weak tokens: the exact
    # tie search ends on a group of equal keys short enough to be ranked
    # lane by lane
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=6000)
    inp = idx_inputs(wl)
    q, w, keys = inp["q"], inp["w"], inp["keys"]
    g = torch.Generator().manual_seed(11)
    n_strong = 980 if stage == "coarse" else 300
    expect = []
    for b in range(2):
        pats = three_level_patterns(q[b].numpy(), w[b].numpy(), keys[b], stage == "coarse")
        perm = torch.randperm(6000, generator=g)
        lvl = torch.full((6000,), 2, dtype=torch.long)
        lvl[perm[:n_strong]] = 0
        lvl[perm[n_strong:n_strong + 50]] = 1
        keys[b] = pats[lvl]
        mid = np.sort(perm[n_strong:n_strong + 50].numpy())[:20]
        expect.append(np.sort(np.concatenate([perm[:n_strong].numpy(), mid])).tolist())
    if stage == "coarse":
        got = run_coarse_case(ls, inp, [6000, 6000], n_strong + 20)
    else:
        got = run_refine_case(ls, inp, [6000, 6000], 6000, n_strong + 20)
    for b in range(2):
        assert got[b].tolist() == expect[b], "request %d" % b


def test_full_candidates_equal_exact_topk_gpu(ls):
    # C = all tokens: the GPU coarse-to-fine result equals the exact top-k
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=4000)
    inp = idx_inputs(wl)
    q, w, keys = inp["q"], inp["w"], inp["keys"]
    cl = torch.tensor([4000, 4000], dtype=torch.int32, device=DEV)
    cand = ls.index_coarse(q.to(DEV), w.to(DEV), ls.pack_coarse(keys.to(DEV)), cl, 4000)
    tk, sc = ls.refine_topk(q.to(DEV), w.to(DEV), keys.to(DEV), cand, cl, 128)
    for b in range(2):
        fine = orc.index_scores(q[b].numpy(), w[b].numpy(), keys[b].numpy(), False)
        ep, es = orc.select_top(fine, np.arange(4000, dtype=np.int32), 128)
        assert np_(tk)[b].tolist() == ep.tolist()
        assert np_(sc)[b].tolist() == es.tolist()


# ---------------------------------------------------------- hot buffer --

def test_hot_gather_parity(ls):
    wl = dataclasses.replace(SHRUNK, batch=3, ctx=3000, topk=200, hot_slots=256, miss_rate=0.3)
    g = torch.Generator().manual_seed(6)
    sel = torch.full((3, 200), -1, dtype=torch.int32)
    counts = [200, 150, 0]
    for b, c in enumerate(counts):
        sel[b, :c] = torch.sort(torch.randperm(3000, generator=g)[:c]).values.to(torch.int32)
    pool = synth.kv_pool(wl, "cpu")
    pos2slot, hot, n_miss = synth.hot_fill(wl, sel, pool, "cpu")
    hot_dev = hot.to(DEV)
    rows, nm = ls.hot_gather(sel.to(DEV), pos2slot.to(DEV), hot_dev, pool.to(DEV), 256)
    rows, nm = np_(rows), np_(nm)
    hot_np = bits(hot).reshape(3, 456, 576).copy()
    pool_np = bits(pool)
    for b in range(3):
        n_sel = counts[b]
        e_rows, e_miss = orc.hot_resolve(np_(sel[b])[:n_sel], np_(pos2slot[b]), 256)
        assert rows[b].tolist() == e_rows.tolist() + [-1] * (200 - n_sel)
        assert nm[b] == len(e_miss) == n_miss[b]
        orc.hot_gather(pool_np[b], e_miss, hot_np[b], 256)
    assert np.array_equal(bits(hot_dev).reshape(3, 456, 576), hot_np)


def test_hot_gather_from_pinned_host_pool(ls):
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=2000, topk=64, hot_slots=64, miss_rate=0.5)
    g = torch.Generator().manual_seed(7)
    sel = torch.stack([torch.sort(torch.randperm(2000, generator=g)[:64]).values
                       for _ in range(2)]).to(torch.int32)
    pool = synth.kv_pool(wl, "cpu", pin=True)
    pos2slot, hot, n_miss = synth.hot_fill(wl, sel, pool, "cpu")
    hot_dev = hot.to(DEV)
    rows, nm = ls.hot_gather(sel.to(DEV), pos2slot.to(DEV), hot_dev, pool, 64)
    torch.cuda.synchronize()
    for b in range(2):
        for i in range(64):
            r = int(np_(rows)[b, i])
            assert torch.equal(hot_dev[b, r].cpu(), pool[b, int(sel[b, i])])
    assert np_(nm).tolist() == n_miss


# ----------------------------------------------------------- attention --

def mla_case(B, Hq, n_rows, K, S, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, 576, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, S + K, 576, generator=g).to(torch.bfloat16)
    rows = torch.full((B, K), -1, dtype=torch.int32)
    for b in range(B):
        rows[b, :n_rows[b]] = torch.randperm(S + K, generator=g)[:n_rows[b]].to(torch.int32)
    return q, kv, rows


def oracle_mla(q, kv, rows, scale):
    B, Hq, _ = q.shape
    outs, lses = [], []
    for b in range(B):
        o, l_ = orc.attention(bits(q[b]), bits(kv[b]).reshape(-1), bits(kv[b]).reshape(-1),
                              np_(rows[b]), scale, 1, 512, 576, 0)
        outs.append(o)
        lses.append(l_)
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("Hq,n_splits", [(128, 0), (128, 1), (128, 3), (64, 0), (16, 2),
                                         (48, 5)])
def test_attention_mla_parity(ls, Hq, n_splits):
    B, K, S = 3, 256, 300
    q, kv, rows = mla_case(B, Hq, [256, 161, 1], K, S, seed=Hq + n_splits)
    scale = 1 / math.sqrt(192)
    kvd = kv.to(DEV)
    out, lse = ls.sparse_attn_decode(q.to(DEV), kvd, kvd, rows.to(DEV), scale, 1, 512, S + K,
                                     576, n_splits=n_splits)
    e_out, e_lse = oracle_mla(q, kv, rows, scale)
    assert_attention_close(out, lse, e_out, e_lse, "mla Hq=%d splits=%d" % (Hq, n_splits))


@pytest.mark.parametrize("n_splits", [9, 11, 16, 40, 64])
def test_attention_mla_parity_many_splits(ls, n_splits):
    # more than eight splits: the combine loads the first 32 at once, then
    # eight at a time (40, 64); a partial last group,
    # a request with no rows at all and one whose rows fill only the first
    # split (the others end with no rows and lse = -inf)
    B, K, S = 3, 512, 300
    q, kv, rows = mla_case(B, 128, [512, 0, 20], K, S, seed=100 + n_splits)
    scale = 1 / math.sqrt(192)
    kvd = kv.to(DEV)
    out, lse = ls.sparse_attn_decode(q.to(DEV), kvd, kvd, rows.to(DEV), scale, 1, 512, S + K,
                                     576, n_splits=n_splits)
    e_out, e_lse = oracle_mla(q, kv, rows, scale)
    assert_attention_close(out, lse, e_out, e_lse, "mla splits=%d" % n_splits)


def test_attention_mla_parity_32_splits(ls):
    # the largest automatic split count (a small batch spread over the
    # CUs): 32 splits of 32 rows, all loaded by the combine in one round
    B, K, S = 2, 1024, 200
    q, kv, rows = mla_case(B, 128, [1024, 700], K, S, seed=132)
    scale = 1 / math.sqrt(192)
    kvd = kv.to(DEV)
    out, lse = ls.sparse_attn_decode(q.to(DEV), kvd, kvd, rows.to(DEV), scale, 1, 512, S + K,
                                     576, n_splits=32)
    e_out, e_lse = oracle_mla(q, kv, rows, scale)
    assert_attention_close(out, lse, e_out, e_lse, "mla splits=32")


def test_attention_mla_all_rows_equal_dense(ls):
    # k >= context: sparse attention over every row equals dense attention
    B, Hq, L = 2, 32, 200
    g = torch.Generator().manual_seed(9)
    q = torch.randn(B, Hq, 576, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, L, 576, generator=g).to(torch.bfloat16)
    rows = torch.arange(L, dtype=torch.int32).repeat(B, 1)
    kvd = kv.to(DEV)
    out, lse = ls.sparse_attn_decode(q.to(DEV), kvd, kvd, rows.to(DEV), 0.07, 1, 512, L, 576)
    qf, kf = q.double(), kv.double()
    s = 0.07 * torch.einsum("bhd,bnd->bhn", qf, kf)
    e_out = torch.einsum("bhn,bnd->bhd", torch.softmax(s, -1), kf[:, :, :512]).numpy()
    e_lse = torch.logsumexp(s, -1).numpy()
    assert_attention_close(out, lse, e_out, e_lse, "dense")


def test_attention_mla_edge_rows(ls):
    B, Hq, K, S = 3, 16, 64, 10
    q, kv, rows = mla_case(B, Hq, [0, 1, 64], K, S, seed=11)
    rows[1, 0] = 4
    kvd = kv.to(DEV)
    out, lse = ls.sparse_attn_decode(q.to(DEV), kvd, kvd, rows.to(DEV), 0.1, 1, 512, S + K, 576,
                                     n_splits=2)
    o = np_(out.float())
    assert np.all(o[0] == 0) and np.all(np.isneginf(np_(lse)[0]))
    # one row: the output is that row's V exactly, lse = its score
    assert torch.equal(out[1].cpu(), kv[1, 4, :512].expand(Hq, 512))
    e_out, e_lse = oracle_mla(q, kv, rows, 0.1)
    assert_attention_close(out[1:], lse[1:], e_out[1:], e_lse[1:], "edge")


def exact_grid_bf16(shape, g, lo=-4, hi=4):
    """bf16 values k/4 for integers k in [lo, hi]: every product of two of
    them, and every partial sum of up to 576 such products, is a multiple of
    1/16 far below 2^20, so an fp32 dot product of them is exact whatever the
    accumulation order (the fp32 rounding of the scores then plays no part)."""
    return (torch.randint(lo, hi + 1, shape, generator=g).float() / 4).to(torch.bfloat16)


def test_attention_mla_score_jump_recomputes(ls):
    # rows after the first 32-row tile score about 90 log2 units above the
    # first tile's maximum (more than the 64 units of headroom of the first
    # pass's base): the kernel must fall back to its exact-max pass.  The
    # values sit on a 1/4 grid so that every score is exact in fp32 and the
    # 1e-4 LSE bound applies at |lse| ~ 60 as it does at ~ 10
    B, Hq, K, S = 2, 128, 256, 64
    g = torch.Generator().manual_seed(77)
    q = exact_grid_bf16((B, Hq, 576), g)
    kv = exact_grid_bf16((B, S + K, 576), g)
    rows = torch.full((B, K), -1, dtype=torch.int32)
    for b, n in enumerate([256, 200]):
        rows[b, :n] = torch.randperm(S + K, generator=g)[:n].to(torch.int32)
    for b in range(B):
        late = rows[b, 40:60].long()
        # only the 64 rope dims grow (32 x a head's own rope query: the head's
        # score jumps by ~850 x scale); V, the first 512 dims, stays on the grid
        kv[b, late, 512:] = (32.0 * q[b, (torch.arange(20) * 5) % Hq, 512:].float()).to(
            torch.bfloat16)
    kvd = kv.to(DEV)
    scale = 1 / math.sqrt(192)
    out, lse = ls.sparse_attn_decode(q.to(DEV), kvd, kvd, rows.to(DEV), scale, 1,
                                     512, S + K, 576, n_splits=1)
    e_out, e_lse = oracle_mla(q, kv, rows, scale)
    # the case does reach the second pass: some head's score exceeds the
    # first tile's maximum by more than 64 log2 units
    qf, kf = q.double(), kv.double()
    for b in range(B):
        n_first = min(32, int((rows[b] >= 0).sum()))
        s = scale / math.log(2) * torch.einsum("hd,nd->hn", qf[b], kf[b, rows[b, :200].long()])
        jump = (s.max(1).values - s[:, :n_first].max(1).values).max()
        assert float(jump) > 64.0, float(jump)
    assert np.isfinite(np_(lse)).all()
    assert_attention_close(out, lse, e_out, e_lse, "score jump")


@pytest.mark.parametrize("Hq,n_kv,D", [(8, 8, 64), (8, 2, 64), (4, 1, 128), (6, 3, 32)])
def test_attention_mha_parity(ls, Hq, n_kv, D):
    B, L, K = 2, 300, 128
    g = torch.Generator().manual_seed(Hq * 7 + n_kv)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    Kc = torch.randn(B, L, n_kv, D, generator=g).to(torch.bfloat16)
    Vc = torch.randn(B, L, n_kv, D, generator=g).to(torch.bfloat16)
    rows = torch.full((B, K), -1, dtype=torch.int32)
    rows[0] = torch.sort(torch.randperm(L, generator=g)[:K]).values.to(torch.int32)
    rows[1, :50] = torch.sort(torch.randperm(L, generator=g)[:50]).values.to(torch.int32)
    out, lse = ls.sparse_attn_decode(q.to(DEV), Kc.to(DEV), Vc.to(DEV), rows.to(DEV), 0.125, n_kv,
                                     D, L, n_kv * D, D)
    e_out, e_lse = [], []
    for b in range(B):
        o, l_ = orc.attention(bits(q[b]), bits(Kc[b]).reshape(-1), bits(Vc[b]).reshape(-1),
                              np_(rows[b]), 0.125, n_kv, D, n_kv * D, D)
        e_out.append(o)
        e_lse.append(l_)
    assert_attention_close(out, lse, np.stack(e_out), np.stack(e_lse), "mha")


def test_attention_mha_many_rows_per_thread(ls):
    # 2000 selected rows: every thread of the generic kernel scores 8 of them;
    # the second request's list ends early (-1 padding)
    B, L, K, Hq, n_kv, D = 2, 3000, 2000, 8, 4, 128
    g = torch.Generator().manual_seed(31)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    Kc = torch.randn(B, L, n_kv, D, generator=g).to(torch.bfloat16)
    Vc = torch.randn(B, L, n_kv, D, generator=g).to(torch.bfloat16)
    rows = torch.full((B, K), -1, dtype=torch.int32)
    rows[0] = torch.sort(torch.randperm(L, generator=g)[:K]).values.to(torch.int32)
    rows[1, :1500] = torch.sort(torch.randperm(L, generator=g)[:1500]).values.to(torch.int32)
    out, lse = ls.sparse_attn_decode(q.to(DEV), Kc.to(DEV), Vc.to(DEV), rows.to(DEV), 0.09, n_kv,
                                     D, L, n_kv * D, D)
    e_out, e_lse = [], []
    for b in range(B):
        o, l_ = orc.attention(bits(q[b]), bits(Kc[b]).reshape(-1), bits(Vc[b]).reshape(-1),
                              np_(rows[b]), 0.09, n_kv, D, n_kv * D, D)
        e_out.append(o)
        e_lse.append(l_)
    assert_attention_close(out, lse, np.stack(e_out), np.stack(e_lse), "mha 2000 rows")


# --------------------------------------------------------- whole step --

def test_decode_step_tiny_mha(ls):
    wl = TINY
    inp = idx_inputs(wl)
    qa = synth.attention_query(wl, "cpu")
    Kc, Vc = synth.kv_cache_mha(wl, "cpu")
    step = ls.DecodeStep(batch=1, max_ctx=wl.ctx, idx_heads=wl.idx_heads, idx_dim=wl.idx_dim,
                         n_cand=wl.n_cand, topk=wl.topk, q_heads=wl.q_heads, qk_dim=wl.qk_dim,
                         v_dim=wl.v_dim, scale=wl.scale, kv_heads=wl.kv_heads,
                         kv_row_stride=wl.kv_heads * wl.qk_dim, kv_head_stride=wl.qk_dim)
    for t in (step.cand, step.topk, step.topk_score, step.out, step.lse):
        poison_(t)
    keys = inp["keys"].to(DEV)
    cl = torch.tensor([wl.ctx], dtype=torch.int32, device=DEV)
    out, lse = step.run(q_idx=inp["q"].to(DEV), w_idx=inp["w"].to(DEV), kc=ls.pack_coarse(keys),
                        k8=keys, ctx_len=cl, q_attn=qa.to(DEV), k_cache=Kc.to(DEV),
                        v_cache=Vc.to(DEV))
    r = orc.decode_request(inp["q"][0].numpy(), inp["w"][0].numpy(), inp["keys"][0].numpy(),
                           wl.ctx, wl.n_cand, wl.topk, bits(qa[0]), wl.scale,
                           k_cache_bits=bits(Kc[0]).reshape(-1),
                           v_cache_bits=bits(Vc[0]).reshape(-1), n_kv_heads=wl.kv_heads,
                           v_dim=wl.v_dim, row_stride=wl.kv_heads * wl.qk_dim,
                           head_stride=wl.qk_dim)
    assert np_(step.cand)[0].tolist() == r["cand"].tolist()
    assert np_(step.topk)[0].tolist() == r["topk"].tolist()
    assert np_(step.topk_score)[0].tolist() == r["topk_score"].tolist()
    assert_attention_close(out, lse, r["out"][None], r["lse"][None], "tiny step")


def mla_step_case(ls, wl, ctx_len, key_rate=None):
    """With key_rate set, the original keys are in pinned host memory behind
    a key cache that misses key_rate of the candidates (k8 rows of cached
    tokens hold unrelated keys)."""
    B = wl.batch
    inp = idx_inputs(wl, ctx_len=ctx_len)
    qa = synth.attention_query(wl, "cpu")
    pool = synth.kv_pool(wl, "cpu")
    sel = []
    for b in range(B):
        cand = oracle_cand(inp["q"][b].numpy(), inp["w"][b].numpy(), inp["keys"][b].numpy(),
                           ctx_len[b], wl.n_cand)
        tk, _ = oracle_topk(inp["q"][b].numpy(), inp["w"][b].numpy(), inp["keys"][b].numpy(),
                            cand, wl.topk)
        sel.append(torch.from_numpy(tk))
    pos2slot, hot, n_miss = synth.hot_fill(wl, torch.stack(sel), pool, "cpu")
    keys = inp["keys"].to(DEV)
    key_cache = {}
    if key_rate is None:
        k8, S = keys, 0
    else:
        S = wl.n_cand
        k8, kp, kcache = cached_key_store(wl, inp, ctx_len, wl.n_cand, key_rate, S, True)
        key_cache = dict(kpos2slot=kp, kcache=kcache)
    step = ls.DecodeStep(batch=B, max_ctx=wl.ctx, idx_heads=wl.idx_heads, idx_dim=wl.idx_dim,
                         n_cand=wl.n_cand, topk=wl.topk, q_heads=wl.q_heads, qk_dim=wl.qk_dim,
                         v_dim=wl.v_dim, scale=wl.scale, hot_slots=wl.hot_slots,
                         keys_on_host=key_rate is not None, key_slots=S)
    for t in (step.cand, step.topk, step.topk_score, step.rows, step.n_miss, step.out, step.lse):
        poison_(t)
    hot_dev = hot.to(DEV)
    cl = torch.tensor(ctx_len, dtype=torch.int32, device=DEV)
    out, lse = step.run(q_idx=inp["q"].to(DEV), w_idx=inp["w"].to(DEV), kc=ls.pack_coarse(keys),
                        k8=k8, ctx_len=cl, q_attn=qa.to(DEV), pos2slot=pos2slot.to(DEV),
                        hot_kv=hot_dev, pool_kv=pool.to(DEV), **key_cache)
    torch.cuda.synchronize()
    for b in range(B):
        hot_b = bits(hot[b]).copy()
        r = orc.decode_request(inp["q"][b].numpy(), inp["w"][b].numpy(), inp["keys"][b].numpy(),
                               ctx_len[b], wl.n_cand, wl.topk, bits(qa[b]), wl.scale,
                               pos2slot=np_(pos2slot[b]), hot_bits=hot_b, pool_bits=bits(pool[b]),
                               v_dim=wl.v_dim, row_stride=wl.qk_dim)
        assert np_(step.cand)[b].tolist() == r["cand"].tolist(), b
        assert np_(step.topk)[b].tolist() == r["topk"].tolist(), b
        assert np_(step.topk_score)[b].tolist() == r["topk_score"].tolist(), b
        assert np_(step.rows)[b].tolist() == r["rows"].tolist(), b
        assert int(np_(step.n_miss)[b]) == r["n_miss"] == n_miss[b], b
        assert np.array_equal(bits(hot_dev[b]), hot_b), b
        assert_attention_close(out[b:b + 1], lse[b:b + 1], r["out"][None], r["lse"][None],
                               "request %d" % b)
    return step


def test_decode_step_shrunk_mla(ls):
    wl = dataclasses.replace(SHRUNK, batch=3, ctx=16384 + 5, n_cand=2048, topk=512,
                             hot_slots=1024, planted=163)
    mla_step_case(ls, wl, [wl.ctx, 9000, 300])


def test_decode_step_host_keys_with_key_cache(ls):
    wl = dataclasses.replace(SHRUNK, batch=3, ctx=8192 + 37, n_cand=1024, topk=256,
                             hot_slots=512)
    mla_step_case(ls, wl, [wl.ctx, 5000, 300], key_rate=0.25)


def test_decode_step_more_than_16384_candidates(ls):
    # the whole step with C > 16384: the block top-k also resolves the hot
    # buffer (rows, miss list, miss count) before the gather and attention
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=40000, n_cand=20000, topk=2048,
                             hot_slots=4096, planted=400)
    mla_step_case(ls, wl, [40000, 23000])


def test_decode_step_many_requests_multi_chunk_emit(ls):
    # 256 requests: each emit workgroup takes both 16384-position chunks of
    # its request in one run; latent rows of 16 elements take the attention
    # without matrix cores and the separate miss gather; most requests are
    # short, every 32nd spans both chunks
    B = 256
    wl = dataclasses.replace(SHRUNK, batch=B, ctx=16400, n_cand=512, topk=64, hot_slots=128,
                             planted=20, idx_heads=4, idx_dim=64, q_heads=8, qk_dim=16, v_dim=16)
    ctx_len = [16400 if b % 32 == 0 else (16384 + 9 if b % 32 == 16 else 200 + (37 * b) % 900)
               for b in range(B)]
    mla_step_case(ls, wl, ctx_len)


def test_decode_step_deterministic(ls):
    wl = dataclasses.replace(SHRUNK, batch=2, ctx=9000, n_cand=1024, topk=256, hot_slots=300)
    inp = idx_inputs(wl)
    qa = synth.attention_query(wl, DEV)
    pool = synth.kv_pool(wl, DEV)
    sel = torch.stack([torch.arange(256, dtype=torch.int32) * 30 for _ in range(2)])
    pos2slot, hot, _ = synth.hot_fill(wl, sel, pool, DEV)
    step = ls.DecodeStep(batch=2, max_ctx=wl.ctx, idx_heads=64, idx_dim=128, n_cand=1024,
                         topk=256, q_heads=128, qk_dim=576, v_dim=512, scale=wl.scale,
                         hot_slots=300)
    keys = inp["keys"].to(DEV)
    kc = ls.pack_coarse(keys)
    cl = torch.tensor([9000, 9000], dtype=torch.int32, device=DEV)
    results = []
    for _ in range(3):
        out, lse = step.run(q_idx=inp["q"].to(DEV), w_idx=inp["w"].to(DEV), kc=kc, k8=keys,
                            ctx_len=cl, q_attn=qa, pos2slot=pos2slot, hot_kv=hot, pool_kv=pool)
        results.append([t.clone() for t in (step.cand, step.topk, step.topk_score, step.rows,
                                            step.n_miss, out.view(torch.int16), lse)])
    for r in results[1:]:
        for a, b_ in zip(results[0], r):
            assert torch.equal(a, b_)
