"""GPU parity of the cache commit (least recently used) and of the new-token
append against the CPU oracle, bit for bit: the standalone commit over
random multi-step sequences and at its maximum sizes, the append (device and
pinned-host stores), and several decode steps in a row with both caches
committing and a new token appended after every step, so that the caches'
contents, hit counts and tables evolve across steps as in serving."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from top_sparse_attention_ls_amd import synth
from tests.gpu_common import np_, bits
from tests.serve_oracle import ServeShadow, empty_tables

pytestmark = pytest.mark.gpu
DEV = "cuda"


def to_dev(p2s, s2p, st):
    return (torch.from_numpy(p2s).to(DEV), torch.from_numpy(s2p).to(DEV),
            torch.from_numpy(st.view(np.int32)).to(DEV))


def check_tables(dev, ref, what):
    p2s, s2p, st = dev
    e_p2s, e_s2p, e_st = ref
    assert np.array_equal(np_(p2s), e_p2s), what + ": pos2slot"
    assert np.array_equal(np_(s2p), e_s2p), what + ": slot2pos"
    assert np.array_equal(np_(st).view(np.uint32), e_st), what + ": stamps"


def commit_sequence(ls, B, L, S, n, steps, seed, now0=1, stamp_hi=0):
    rng = np.random.default_rng(seed)
    p2s, s2p, st = empty_tables(B, L, S)
    if stamp_hi:
        # a cache already in use: every slot occupied, stamps spread over the
        # whole 32-bit range below now0 (all three radix digits vary)
        for b in range(B):
            pos = rng.choice(L, size=S, replace=False).astype(np.int32)
            s2p[b] = pos
            p2s[b, pos] = np.arange(S, dtype=np.int32)
            st[b] = rng.integers(0, stamp_hi, S, dtype=np.uint64).astype(np.uint32)
            st[b, rng.choice(S, size=S // 8, replace=False)] = st[b, 0]  # equal stamps
    dev = to_dev(p2s, s2p, st)
    hot_set = [rng.choice(L, size=max(n, L // 6), replace=False) for _ in range(B)]
    for k in range(steps):
        now = now0 + k
        ent = np.full((B, n), -1, np.int32)
        for b in range(B):
            pick = np.where(rng.random(n) < 0.6, rng.choice(hot_set[b], n),
                            rng.integers(0, L, n))
            u = np.unique(pick).astype(np.int32)[: n - (b % 3)]
            ent[b, :len(u)] = u
        dst, n_ins = ls.cache_commit(torch.from_numpy(ent).to(DEV), *dev, now)
        for b in range(B):
            e_dst, e_n = orc.cache_commit(ent[b], S, now, p2s[b], s2p[b], st[b])
            assert np_(dst)[b].tolist() == e_dst.tolist(), (k, b, "dst")
            assert int(np_(n_ins)[b]) == e_n, (k, b, "inserted")
        check_tables(dev, (p2s, s2p, st), "step %d" % k)


def test_cache_commit_multi_step(ls):
    commit_sequence(ls, B=3, L=5000, S=700, n=300, steps=8, seed=1)


def test_cache_commit_more_misses_than_slots(ls):
    commit_sequence(ls, B=2, L=3000, S=100, n=250, steps=4, seed=2)


def test_cache_commit_stamps_over_the_whole_range(ls):
    commit_sequence(ls, B=2, L=40000, S=4096, n=2048, steps=3, seed=3, now0=0xFFFFFF00,
                    stamp_hi=0xFFFFFF00)


def test_cache_commit_maximum_sizes(ls):
    commit_sequence(ls, B=2, L=70000, S=16384, n=16384, steps=2, seed=4)


@pytest.mark.parametrize("host", [False, True], ids=["device", "pinned-host"])
def test_append_token(ls, host):
    B, L, D, row = 3, 50, 128, 576
    g = torch.Generator().manual_seed(9)
    k8 = torch.randint(-128, 128, (B, L, D), generator=g, dtype=torch.int32).to(torch.int8)
    pool = torch.randn(B, L, row, generator=g).to(torch.bfloat16)
    kc = torch.from_numpy(orc.pack_coarse(k8.numpy()))
    ctx = [0, 17, L]                      # empty, partial, full (left unchanged)
    new_k = torch.randint(-128, 128, (B, D), generator=g, dtype=torch.int32).to(torch.int8)
    new_k[0, :] = torch.arange(-128, 128, 2, dtype=torch.int32)[:D].to(torch.int8)
    new_kv = torch.randn(B, row, generator=g).to(torch.bfloat16)
    k8_s = k8.pin_memory() if host else k8.to(DEV)
    pool_s = pool.pin_memory() if host else pool.to(DEV)
    kc_d = kc.to(DEV)
    cl = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    ls.append_token(new_k.to(DEV), k8_s, kc_d, cl, new_kv=new_kv.to(DEV), pool=pool_s)
    torch.cuda.synchronize()
    e_k8, e_pool = k8.clone(), pool.clone()
    for b in range(B):
        if ctx[b] < L:
            e_k8[b, ctx[b]] = new_k[b]
            e_pool[b, ctx[b]] = new_kv[b]
    assert torch.equal(k8_s.cpu(), e_k8)
    assert np.array_equal(bits(pool_s), bits(e_pool))
    assert np.array_equal(np_(kc_d), orc.pack_coarse(e_k8.numpy()))
    assert np_(cl).tolist() == [1, 18, L]


@pytest.mark.parametrize("keys_host,pool_host", [(True, False), (False, True)],
                         ids=["host-keys", "host-pool"])
def test_decode_steps_with_commits_and_append(ls, keys_host, pool_host):
    wl = dataclasses.replace(synth.WORKLOADS["decode-128k-b32"], name="commit-steps", batch=3,
                             ctx=6000, n_cand=1024, topk=256, planted=60, hot_slots=400,
                             keys_on_host=True, key_slots=1500)
    B, L, H, D, C, K, S, SK = (wl.batch, wl.ctx, wl.idx_heads, wl.idx_dim, wl.n_cand, wl.topk,
                               wl.hot_slots, wl.key_slots)
    ctx = [L - 10, 4000, 0]           # full-ish, partial, empty (grows by the appends)
    inp = synth.indexer_inputs(wl, "cpu", ctx_len=ctx)
    q, w, keys = inp["q"], inp["w"], inp["keys"].clone()
    pool = synth.kv_pool(wl, "cpu")
    q_attn = synth.attention_query(wl, "cpu")
    row = wl.qk_dim

    # both caches start empty; the oracle's state is kept by the shadow
    shadow = ServeShadow(wl, keys, pool, q_attn, ctx)
    p2s, s2p, st = empty_tables(B, L, S)
    kp2s, ks2p, kst = empty_tables(B, L, SK)
    d_hot = torch.zeros((B, S + K, row), dtype=torch.bfloat16, device=DEV)
    d_tab = to_dev(p2s, s2p, st)
    d_ktab = to_dev(kp2s, ks2p, kst)
    d_kcache = torch.zeros((B, SK, D), dtype=torch.int8, device=DEV)
    # the key store and the pool where the case puts them (the names keep
    # the host-keys case's)
    k8_host = keys.pin_memory() if keys_host else keys.to(DEV)
    pool_d = pool.pin_memory() if pool_host else pool.to(DEV)
    kc_d = ls.pack_coarse(keys.to(DEV))
    cl_d = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    step = ls.DecodeStep(batch=B, max_ctx=L, idx_heads=H, idx_dim=D, n_cand=C, topk=K,
                         q_heads=wl.q_heads, qk_dim=wl.qk_dim, v_dim=wl.v_dim, scale=wl.scale,
                         hot_slots=S, keys_on_host=keys_host, key_slots=SK, commit_hot=True,
                         commit_keys=True, pool_on_host=pool_host)
    g = torch.Generator().manual_seed(77)
    for k in range(5):
        now = k + 1
        if k:
            q = synth.drift_query(q, 0.15, torch.Generator().manual_seed(100 + k), "cpu")
        print("[commit-steps] step %d" % k, flush=True)
        out, lse = step.run(q_idx=q.to(DEV), w_idx=w.to(DEV), kc=kc_d, k8=k8_host, ctx_len=cl_d,
                            q_attn=q_attn.to(DEV), pos2slot=d_tab[0], hot_kv=d_hot,
                            pool_kv=pool_d, kpos2slot=d_ktab[0], kcache=d_kcache,
                            slot2pos=d_tab[1], stamp=d_tab[2], kslot2pos=d_ktab[1],
                            kstamp=d_ktab[2], now=now)
        torch.cuda.synchronize()
        shadow.step(step, out, lse, q, w, now, "step %d" % k)
        shadow.check_state(d_hot, d_tab, d_ktab, d_kcache, "step %d" % k)
        # the step's new token, appended on both sides
        new_k = synth.int8_normal((B, D), 24.0, g, "cpu")
        new_kv = torch.randn(B, row, generator=g).to(torch.bfloat16)
        ls.append_token(new_k.to(DEV), k8_host, kc_d, cl_d, new_kv=new_kv.to(DEV), pool=pool_d)
        torch.cuda.synchronize()
        shadow.append(new_k, new_kv)
        shadow.check_stores(k8_host, pool_d, cl_d, "append %d" % k)
        assert np.array_equal(np_(kc_d), orc.pack_coarse(shadow.keys.numpy())), k
    # the drifting query keeps part of its selection from step to step
    assert shadow.hits > 0


def serve_state(ls, wl, B, dev):
    L, D, S, SK, K, row = wl.ctx, wl.idx_dim, wl.hot_slots, wl.key_slots, wl.topk, wl.qk_dim
    inp = synth.indexer_inputs(wl, dev)
    g = torch.Generator(device=dev).manual_seed(3)
    return dict(
        q=inp["q"], w=inp["w"], kc=ls.pack_coarse(inp["keys"]), k8=inp["keys"].cpu().pin_memory(),
        pool=synth.kv_pool(wl, dev), q_attn=synth.attention_query(wl, dev),
        ctx_len=torch.tensor([L - 9, L // 2, 1000, L - 1][:B], dtype=torch.int32, device=dev),
        new_k=synth.int8_normal((B, D), 24.0, g, dev), new_kv=synth.bf16_normal((B, row), g, dev),
        hot=torch.zeros((B, S + K, row), dtype=torch.bfloat16, device=dev),
        p2s=torch.full((B, L), -1, dtype=torch.int32, device=dev),
        s2p=torch.full((B, S), -1, dtype=torch.int32, device=dev),
        st=torch.zeros((B, S), dtype=torch.int32, device=dev),
        kp2s=torch.full((B, L), -1, dtype=torch.int32, device=dev),
        ks2p=torch.full((B, SK), -1, dtype=torch.int32, device=dev),
        kst=torch.zeros((B, SK), dtype=torch.int32, device=dev),
        kcache=torch.zeros((B, SK, D), dtype=torch.int8, device=dev))


class Joined:
    """The step outputs of consecutive request ranges, as one batch."""

    def __init__(self, parts):
        for name in ("cand", "topk", "topk_score", "rows", "n_miss", "n_key_miss"):
            setattr(self, name, torch.cat([getattr(p_, name) for p_ in parts]))


def test_micro_batches_on_two_streams_match_one_batch(ls):
    # the serving loop's overlap pattern: the batch split into two request
    # ranges (views into the same state, the pinned keys included), each with
    # its own step on its own stream, the second starting each step once the
    # first has selected its candidates; every table, cache row, output and
    # appended token must equal the oracle's serving loop stepped alongside,
    # and one step over the whole batch
    wl = dataclasses.replace(synth.WORKLOADS["decode-128k-b32"], name="mb", batch=4, ctx=6000,
                             n_cand=1024, topk=256, planted=60, hot_slots=400, key_slots=1500)
    B, Bm = 4, 2
    one, two = serve_state(ls, wl, B, DEV), serve_state(ls, wl, B, DEV)

    def make_step(batch):
        return ls.DecodeStep(batch=batch, max_ctx=wl.ctx, idx_heads=wl.idx_heads,
                             idx_dim=wl.idx_dim, n_cand=wl.n_cand, topk=wl.topk,
                             q_heads=wl.q_heads, qk_dim=wl.qk_dim, v_dim=wl.v_dim, scale=wl.scale,
                             hot_slots=wl.hot_slots, keys_on_host=True, key_slots=wl.key_slots,
                             commit_hot=True, commit_keys=True, n_splits=4)

    def run(step, x, now, events=None):
        step.run(q_idx=x["q"], w_idx=x["w"], kc=x["kc"], k8=x["k8"], ctx_len=x["ctx_len"],
                 q_attn=x["q_attn"], pos2slot=x["p2s"], hot_kv=x["hot"], pool_kv=x["pool"],
                 kpos2slot=x["kp2s"], kcache=x["kcache"], slot2pos=x["s2p"], stamp=x["st"],
                 kslot2pos=x["ks2p"], kstamp=x["kst"], now=now, events=events)
        ls.append_token(x["new_k"], x["k8"], x["kc"], x["ctx_len"], new_kv=x["new_kv"],
                        pool=x["pool"])

    whole = make_step(B)
    parts = [make_step(Bm), make_step(Bm)]
    views = [{k: v[m * Bm:(m + 1) * Bm] for k, v in two.items()} for m in range(2)]
    shadow = ServeShadow(wl, two["k8"], two["pool"], two["q_attn"], np_(two["ctx_len"]).tolist())
    q_cpu, w_cpu = two["q"].cpu(), two["w"].cpu()
    side = torch.cuda.Stream()
    sel = torch.cuda.Event()
    for k in range(4):
        now = k + 1
        run(whole, one, now)
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        ev = [None] * ls.STEP_EVENTS
        ev[2] = sel
        run(parts[0], views[0], now, ev)
        with torch.cuda.stream(side):
            side.wait_event(sel)
            run(parts[1], views[1], now)
        main.wait_stream(side)
        torch.cuda.synchronize()
        # the two ranges against the oracle
        got_out = torch.cat([p_.out for p_ in parts])
        got_lse = torch.cat([p_.lse for p_ in parts])
        shadow.step(Joined(parts), got_out, got_lse, q_cpu, w_cpu, now, "step %d" % k)
        shadow.check_state(two["hot"], (two["p2s"], two["s2p"], two["st"]),
                           (two["kp2s"], two["ks2p"], two["kst"]), two["kcache"], "step %d" % k)
        shadow.append(two["new_k"].cpu(), two["new_kv"].cpu())
        shadow.check_stores(two["k8"], two["pool"], two["ctx_len"], "append %d" % k)
        # and against one step over the whole batch
        for name in ("cand", "topk", "topk_score", "rows", "n_miss", "n_key_miss", "lse"):
            got = torch.cat([getattr(p_, name) for p_ in parts])
            assert torch.equal(got, getattr(whole, name)), (k, name)
        got_out = torch.cat([p_.out for p_ in parts])
        assert torch.equal(got_out.view(torch.int16), whole.out.view(torch.int16)), k
        for key in ("hot", "p2s", "s2p", "st", "kp2s", "ks2p", "kst", "kcache", "kc", "ctx_len",
                    "pool", "k8"):
            a, b_ = one[key], two[key]
            if a.dtype == torch.bfloat16:
                a, b_ = a.view(torch.int16), b_.view(torch.int16)
            assert torch.equal(a, b_), (k, key)
