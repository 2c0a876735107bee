"""GPU parity at the served workloads' full sizes, in the launch configuration
the benchmark times (one DecodeStep call over the whole batch, automatic
split count), against the CPU oracle on every request (the oracle runs on a
pool of host threads).

The hot buffer is laid out from the generator's planted positions (all of
them resident, the remaining slots random), which the HIP path never sees,
so no oracle input comes from the GPU.  On every request, sampled or not,
the test also checks what holds at any size: ascending, in-range, unique
positions; selected scores equal to the oracle's exact score of those
positions; hot-buffer rows and miss list consistent with the slot table; the
gathered rows byte-equal to the pool rows.

With the original keys on the host, the key cache is laid out the same way
(the planted positions cached, the remaining rows random tokens), so the
candidates' keys come from both the cache and the host store."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from top_sparse_attention_ls_amd import synth
from tests.gpu_common import (np_, bits, assert_attention_close, oracle_cand, oracle_topk,
                              parallel_map)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_full(ls, name, sample):
    wl = synth.WORKLOADS[name]
    B, L = wl.batch, wl.ctx
    print("[fullsize] %s: building inputs" % name, flush=True)
    inp = synth.indexer_inputs(wl, DEV)
    qa = synth.attention_query(wl, DEV)
    pool = synth.kv_pool(wl, DEV, pin=wl.pool_on_host, gen_device=DEV)
    width = max(int(p.numel()) for p in inp["planted"])
    planted = torch.full((B, width), -1, dtype=torch.int32)
    for b, p in enumerate(inp["planted"]):
        planted[b, :p.numel()] = p.to("cpu", torch.int32)
    pos2slot, hot, _ = synth.hot_fill(wl, planted, pool, DEV, miss_rate=0.0, scratch=wl.topk)
    hot0 = hot.clone()
    keys = inp["keys"]
    kc = ls.pack_coarse(keys)
    ctx_len = torch.full((B,), L, dtype=torch.int32, device=DEV)
    key_cache, k8 = {}, keys
    if wl.key_slots:
        kp, kcache, _ = synth.key_cache_fill(wl, planted, keys, DEV, miss_rate=0.0)
        key_cache = dict(kpos2slot=kp, kcache=kcache)
    if wl.keys_on_host:
        k8 = keys.to("cpu").pin_memory()
    step = ls.DecodeStep(batch=B, max_ctx=L, idx_heads=wl.idx_heads, idx_dim=wl.idx_dim,
                         n_cand=wl.n_cand, topk=wl.topk, q_heads=wl.q_heads, qk_dim=wl.qk_dim,
                         v_dim=wl.v_dim, scale=wl.scale, hot_slots=wl.hot_slots,
                         pool_on_host=wl.pool_on_host, keys_on_host=wl.keys_on_host,
                         key_slots=wl.key_slots, device=DEV)
    print("[fullsize] %s: step" % name, flush=True)
    out, lse = step.run(q_idx=inp["q"], w_idx=inp["w"], kc=kc, k8=k8, ctx_len=ctx_len,
                        q_attn=qa, pos2slot=pos2slot, hot_kv=hot, pool_kv=pool, **key_cache)
    torch.cuda.synchronize()

    cand, topk, score = np_(step.cand), np_(step.topk), np_(step.topk_score)
    rows, n_miss = np_(step.rows), np_(step.n_miss)
    p2s = np_(pos2slot)
    S, K = wl.hot_slots, wl.topk
    for b in range(B):
        c = cand[b][cand[b] >= 0]
        assert len(c) == min(wl.n_cand, L), (b, len(c))
        assert (np.diff(c) > 0).all() and c[-1] < L, (b, "candidates not ascending/in range")
        t = topk[b][topk[b] >= 0]
        assert len(t) == min(K, len(c)), (b, len(t), "selected count")
        assert (np.diff(t) > 0).all(), (b, "top-k not ascending", np.where(np.diff(t) <= 0)[0][:8])
        assert np.isin(t, c).all(), (b, "top-k outside the candidates")
        exact = orc.index_scores_at(np_(inp["q"][b]), np_(inp["w"][b]), np_(keys[b]),
                                    t.astype(np.int32), False)
        bad = np.where(score[b][:len(t)] != exact)[0]
        assert len(bad) == 0, (b, "scores differ at", bad[:8], score[b][bad[:4]], exact[bad[:4]])
        slot = p2s[b][t]
        miss = slot < 0
        assert n_miss[b] == miss.sum(), (b, int(n_miss[b]), int(miss.sum()), "miss count")
        bad = np.where(rows[b][:len(t)][~miss] != slot[~miss])[0]
        assert len(bad) == 0, (b, "hit rows differ at", bad[:8])
        bad = np.where(rows[b][:len(t)][miss] != S + np.arange(miss.sum()))[0]
        assert len(bad) == 0, (b, "miss rows differ at", bad[:8], rows[b][:len(t)][miss][bad[:4]])
        got = bits(hot[b, S:S + int(miss.sum())])
        assert np.array_equal(got, bits(pool[b].index_select(
            0, torch.from_numpy(t[miss]).to(pool.device, torch.int64)))), b

    def oracle_of(b):
        hot_b = bits(hot0[b]).copy()
        r = orc.decode_request(np_(inp["q"][b]), np_(inp["w"][b]), np_(keys[b]), L, wl.n_cand,
                               wl.topk, bits(qa[b]), wl.scale, pos2slot=p2s[b],
                               hot_bits=hot_b, pool_bits=bits(pool[b]))
        return b, r, hot_b

    print("[fullsize] %s: oracle on %d requests (host threads)" % (name, len(sample)),
          flush=True)
    for b, r, hot_b in parallel_map(oracle_of, sample):
        bad = np.where(cand[b] != r["cand"])[0]
        assert len(bad) == 0, (b, "candidates differ at", bad[:8], cand[b][bad[:4]], r["cand"][bad[:4]])
        bad = np.where(topk[b] != r["topk"])[0]
        assert len(bad) == 0, (b, "top-k differs at", bad[:8], topk[b][bad[:4]], r["topk"][bad[:4]])
        assert score[b].tolist() == r["topk_score"].tolist(), b
        assert rows[b].tolist() == r["rows"].tolist(), b
        assert int(n_miss[b]) == r["n_miss"], b
        assert np.array_equal(bits(hot[b]), hot_b), b
        assert_attention_close(out[b:b + 1], lse[b:b + 1], r["out"][None], r["lse"][None],
                               "%s request %d" % (name, b))


@pytest.mark.timeout(300)
def test_fullsize_decode_128k_b32(ls):
    run_full(ls, "decode-128k-b32", sample=range(32))


@pytest.mark.timeout(300)
def test_fullsize_decode_128k_b32_host_keys_with_key_cache(ls):
    run_full(ls, "decode-128k-b32-hostkeys", sample=range(32))


@pytest.mark.timeout(300)
def test_fullsize_decode_16k_b192_pinned_host_pool(ls):
    run_full(ls, "decode-16k-b192", sample=range(192))


@pytest.mark.timeout(300)
def test_fullsize_decode_950k_b4(ls):
    run_full(ls, "decode-950k-b4", sample=range(4))


@pytest.mark.timeout(300)
def test_fullsize_serving_steps_keep_the_caches_coherent(ls):
    # the serving workload at full size, as the benchmark runs it (both caches
    # committing from empty, one token appended per step): after each step
    # the tables are coherent, every cached row holds its token's bytes, the
    # stamps are this step's or older, and request 5's candidates, selection
    # and commits equal the oracle's, stepped alongside from the generator's
    # inputs
    wl = synth.WORKLOADS["decode-128k-b32-serve"]
    B, L, D, C, K, S, SK, row = (wl.batch, wl.ctx, wl.idx_dim, wl.n_cand, wl.topk, wl.hot_slots,
                                 wl.key_slots, wl.qk_dim)
    print("[fullsize] serve: building inputs", flush=True)
    inp = synth.indexer_inputs(wl, DEV)
    keys = inp["keys"]
    kc = ls.pack_coarse(keys)
    k8 = keys.to("cpu").pin_memory()
    pool = synth.kv_pool(wl, DEV, gen_device=DEV)
    qa = synth.attention_query(wl, DEV)
    ctx_len = torch.full((B,), L - 16, dtype=torch.int32, device=DEV)
    hot = torch.zeros((B, S + K, row), dtype=torch.bfloat16, device=DEV)
    p2s = torch.full((B, L), -1, dtype=torch.int32, device=DEV)
    s2p = torch.full((B, S), -1, dtype=torch.int32, device=DEV)
    st = torch.zeros((B, S), dtype=torch.int32, device=DEV)
    kp2s = torch.full((B, L), -1, dtype=torch.int32, device=DEV)
    ks2p = torch.full((B, SK), -1, dtype=torch.int32, device=DEV)
    kst = torch.zeros((B, SK), dtype=torch.int32, device=DEV)
    kcache = torch.zeros((B, SK, D), dtype=torch.int8, device=DEV)
    step = ls.DecodeStep(batch=B, max_ctx=L, idx_heads=wl.idx_heads, idx_dim=D, n_cand=C,
                         topk=K, q_heads=wl.q_heads, qk_dim=wl.qk_dim, v_dim=wl.v_dim,
                         scale=wl.scale, hot_slots=S, keys_on_host=True, key_slots=SK,
                         commit_hot=True, commit_keys=True, device=DEV)
    g = synth.generator(wl.seed, 100, 0, DEV)
    q = inp["q"]
    r, ctx_r = 5, L - 16
    o_hot = [np_(p2s[r]).copy(), np_(s2p[r]).copy(), np_(st[r]).view(np.uint32).copy()]
    o_key = [np_(kp2s[r]).copy(), np_(ks2p[r]).copy(), np_(kst[r]).view(np.uint32).copy()]
    for k in range(3):
        now = k + 1
        print("[fullsize] serve: step %d" % k, flush=True)
        step.run(q_idx=q, w_idx=inp["w"], kc=kc, k8=k8, ctx_len=ctx_len, q_attn=qa,
                 pos2slot=p2s, hot_kv=hot, pool_kv=pool, kpos2slot=kp2s, kcache=kcache,
                 slot2pos=s2p, stamp=st, kslot2pos=ks2p, kstamp=kst, now=now)
        torch.cuda.synchronize()
        # the oracle's step of request r: candidates, selection, both commits
        qr, wr, kr = np_(q[r]), np_(inp["w"][r]), np_(keys[r])
        e_cand = oracle_cand(qr, wr, kr, ctx_r, C)
        e_tk, _ = oracle_topk(qr, wr, kr, e_cand, K)
        assert np_(step.cand)[r].tolist() == e_cand.tolist(), (k, "cand")
        assert np_(step.topk)[r].tolist() == e_tk.tolist(), (k, "topk")
        e_dst, _ = orc.cache_commit(e_tk, S, now, *o_hot)
        orc.cache_commit(e_cand, SK, now, *o_key)
        assert np.array_equal(np_(p2s[r]), o_hot[0]) and np.array_equal(np_(s2p[r]), o_hot[1])
        assert np.array_equal(np_(st[r]).view(np.uint32), o_hot[2])
        assert np.array_equal(np_(kp2s[r]), o_key[0]) and np.array_equal(np_(ks2p[r]), o_key[1])
        assert np.array_equal(np_(kst[r]).view(np.uint32), o_key[2])
        sel = e_tk
        got_rows = np_(step.rows)[r]
        for i in range(len(sel)):
            if sel[i] >= 0 and e_dst[i] >= 0:
                assert got_rows[i] == e_dst[i], (k, i)
        # every request: coherent tables, cached rows equal to their tokens'
        for b in range(B):
            for tab, s2p_, cache, src in ((p2s, s2p, hot, pool), (kp2s, ks2p, kcache, keys)):
                sp = s2p_[b]
                occ = torch.nonzero(sp >= 0).flatten()
                pos = sp[occ].long()
                assert torch.equal(tab[b, pos], occ.to(torch.int32)), (k, b, "table")
                assert int((tab[b] >= 0).sum()) == occ.numel(), (k, b, "extra entries")
                assert torch.equal(cache[b, occ], src[b, pos]), (k, b, "cached rows")
        assert int(st.max()) == now and int(kst.max()) == now
        new_k = synth.int8_normal((B, D), 24.0, g, DEV)
        new_kv = synth.bf16_normal((B, row), g, DEV)
        pos_new = ctx_len.long().clone()
        ls.append_token(new_k, k8, kc, ctx_len, new_kv=new_kv, pool=pool)
        keys[torch.arange(B, device=DEV), pos_new] = new_k
        ctx_r += 1
        q = synth.drift_query(q, wl.serve_drift, g, DEV)
    torch.cuda.synchronize()
    assert torch.equal(k8, keys.cpu())
