"""The decode step captured in a HIP graph.  The step only enqueues kernels
(no allocation, no memset, no host synchronisation), so it can be captured;
every replay -- with eager steps and synchronisations in between -- must give
the eager step's results bit for bit, including the hot-buffer scratch rows
it writes and the workspace it leaves cleared for the next call; the
single-request MHA step's replays are also checked against the oracle.  The
captured layer stack of the serving loop is also stepped against the
oracle's serving loop after every replay."""
import dataclasses

import pytest
import torch

from oracle import oracle as orc
from top_sparse_attention_ls_amd import synth
from tests.gpu_common import np_, bits, poison_, assert_attention_close
from tests.serve_oracle import ServeShadow

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_decode_step_graph_replays_match_eager(ls):
    wl = dataclasses.replace(synth.WORKLOADS["decode-128k-b32"], name="graph-16k", batch=3,
                             ctx=16384 + 7, n_cand=2048, topk=512, hot_slots=1024, planted=163)
    inp = synth.indexer_inputs(wl, DEV)
    qa = synth.attention_query(wl, DEV)
    pool = synth.kv_pool(wl, DEV)
    g = torch.Generator().manual_seed(7)
    sel = torch.stack([torch.randperm(wl.ctx, generator=g)[:wl.topk].sort().values.to(torch.int32)
                       for _ in range(wl.batch)])
    pos2slot, hot, _ = synth.hot_fill(wl, sel, pool, DEV)
    keys = inp["keys"]
    step = ls.DecodeStep(batch=wl.batch, max_ctx=wl.ctx, idx_heads=wl.idx_heads,
                         idx_dim=wl.idx_dim, n_cand=wl.n_cand, topk=wl.topk, q_heads=wl.q_heads,
                         qk_dim=wl.qk_dim, v_dim=wl.v_dim, scale=wl.scale,
                         hot_slots=wl.hot_slots, device=DEV)
    args = dict(q_idx=inp["q"], w_idx=inp["w"], kc=ls.pack_coarse(keys), k8=keys,
                ctx_len=torch.tensor([wl.ctx, 9000, 1], dtype=torch.int32, device=DEV),
                q_attn=qa, pos2slot=pos2slot, hot_kv=hot, pool_kv=pool)

    def state(out, lse):
        return [t.clone() for t in (step.cand, step.topk, step.topk_score, step.rows,
                                    step.n_miss, out.view(torch.int16), lse, hot.view(torch.int16))]

    out, lse = step.run(**args)
    torch.cuda.synchronize()
    ref = state(out, lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run(**args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gout, glse = step.run(**args)
    torch.cuda.synchronize()

    for i in range(4):
        for t in (step.cand, step.topk, step.rows, gout, glse):
            t.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        got = state(gout, glse)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), "replay %d differs from the eager step" % i
        out, lse = step.run(**args)  # eager work between the replays
        torch.cuda.synchronize()
        for a, b in zip(ref, state(out, lse)):
            assert torch.equal(a, b), "eager step after replay %d differs" % i


def test_tiny_mha_step_graph_replays_match_oracle(ls):
    # the single-request 4K step (generic MHA attention, no hot buffer) as the
    # bench replays it: every replay, with eager steps between, against the
    # oracle's request and bit for bit against the eager step
    wl = synth.WORKLOADS["tiny-4k"]
    inp = synth.indexer_inputs(wl, "cpu")
    qa = synth.attention_query(wl, "cpu")
    Kc, Vc = synth.kv_cache_mha(wl, "cpu")
    step = ls.DecodeStep(batch=1, max_ctx=wl.ctx, idx_heads=wl.idx_heads, idx_dim=wl.idx_dim,
                         n_cand=wl.n_cand, topk=wl.topk, q_heads=wl.q_heads, qk_dim=wl.qk_dim,
                         v_dim=wl.v_dim, scale=wl.scale, kv_heads=wl.kv_heads,
                         kv_row_stride=wl.kv_heads * wl.qk_dim, kv_head_stride=wl.qk_dim)
    keys = inp["keys"].to(DEV)
    args = dict(q_idx=inp["q"].to(DEV), w_idx=inp["w"].to(DEV), kc=ls.pack_coarse(keys), k8=keys,
                ctx_len=torch.tensor([wl.ctx], dtype=torch.int32, device=DEV),
                q_attn=qa.to(DEV), k_cache=Kc.to(DEV), v_cache=Vc.to(DEV))
    r = orc.decode_request(inp["q"][0].numpy(), inp["w"][0].numpy(), inp["keys"][0].numpy(),
                           wl.ctx, wl.n_cand, wl.topk, bits(qa[0]), wl.scale,
                           k_cache_bits=bits(Kc[0]).reshape(-1),
                           v_cache_bits=bits(Vc[0]).reshape(-1), n_kv_heads=wl.kv_heads,
                           v_dim=wl.v_dim, row_stride=wl.kv_heads * wl.qk_dim,
                           head_stride=wl.qk_dim)

    def check(out, lse, what):
        assert np_(step.cand)[0].tolist() == r["cand"].tolist(), what
        assert np_(step.topk)[0].tolist() == r["topk"].tolist(), what
        assert np_(step.topk_score)[0].tolist() == r["topk_score"].tolist(), what
        assert_attention_close(out, lse, r["out"][None], r["lse"][None], what)

    out, lse = step.run(**args)
    torch.cuda.synchronize()
    check(out, lse, "eager step")
    ref = [t.clone() for t in (step.cand, step.topk, step.topk_score, out.view(torch.int16), lse)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run(**args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gout, glse = step.run(**args)
    torch.cuda.synchronize()

    for i in range(3):
        for t in (step.cand, step.topk, step.topk_score, gout, glse):
            poison_(t)
        graph.replay()
        torch.cuda.synchronize()
        check(gout, glse, "replay %d" % i)
        got = (step.cand, step.topk, step.topk_score, gout.view(torch.int16), glse)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), "replay %d differs from the eager step" % i
        out, lse = step.run(**args)  # eager work between the replays
        torch.cuda.synchronize()
        check(out, lse, "eager step after replay %d" % i)


def serving_layer(ls, wl, seed, dev):
    lw = dataclasses.replace(wl, seed=seed)
    B, L, D, S, SK, K, row = (lw.batch, lw.ctx, lw.idx_dim, lw.hot_slots, lw.key_slots, lw.topk,
                              lw.qk_dim)
    inp = synth.indexer_inputs(lw, dev)
    g = torch.Generator(device=dev).manual_seed(seed)
    return dict(
        q=inp["q"], w=inp["w"], kc=ls.pack_coarse(inp["keys"]), k8=inp["keys"].cpu().pin_memory(),
        pool=synth.kv_pool(lw, dev), q_attn=synth.attention_query(lw, dev),
        ctx_len=torch.tensor([L - 8, L // 2], dtype=torch.int32, device=dev),
        new_k=synth.int8_normal((B, D), 24.0, g, dev), new_kv=synth.bf16_normal((B, row), g, dev),
        hot=torch.zeros((B, S + K, row), dtype=torch.bfloat16, device=dev),
        p2s=torch.full((B, L), -1, dtype=torch.int32, device=dev),
        s2p=torch.full((B, S), -1, dtype=torch.int32, device=dev),
        st=torch.zeros((B, S), dtype=torch.int32, device=dev),
        kp2s=torch.full((B, L), -1, dtype=torch.int32, device=dev),
        ks2p=torch.full((B, SK), -1, dtype=torch.int32, device=dev),
        kst=torch.zeros((B, SK), dtype=torch.int32, device=dev),
        kcache=torch.zeros((B, SK, D), dtype=torch.int8, device=dev),
        step=ls.DecodeStep(batch=B, max_ctx=L, idx_heads=lw.idx_heads, idx_dim=D,
                           n_cand=lw.n_cand, topk=K, q_heads=lw.q_heads, qk_dim=lw.qk_dim,
                           v_dim=lw.v_dim, scale=lw.scale, hot_slots=S, keys_on_host=True,
                           key_slots=SK, commit_hot=True, commit_keys=True, device=dev))


def test_layer_stack_serving_graph_matches_eager(ls):
    # two layers, each with its own caches committing every step and a token
    # appended per step; the stamp comes from a device counter that the token
    # step advances, so one captured token step replays correctly step after
    # step.  The graph runs on one copy of the state, the eager steps on an
    # identical copy; after every replay (with eager work and synchronisation
    # in between) both copies must agree bit for bit.
    wl = dataclasses.replace(synth.WORKLOADS["decode-128k-b32"], name="stack", batch=2,
                             ctx=8192, n_cand=1024, topk=256, planted=82, hot_slots=600,
                             key_slots=1500)
    copies = [[serving_layer(ls, wl, 500 + l, DEV) for l in range(2)] for _ in range(2)]
    nows = [torch.ones((1,), dtype=torch.int32, device=DEV) for _ in range(2)]

    def token_step(layers, now):
        for x in layers:
            x["step"].run(q_idx=x["q"], w_idx=x["w"], kc=x["kc"], k8=x["k8"],
                          ctx_len=x["ctx_len"], q_attn=x["q_attn"], pos2slot=x["p2s"],
                          hot_kv=x["hot"], pool_kv=x["pool"], kpos2slot=x["kp2s"],
                          kcache=x["kcache"], slot2pos=x["s2p"], stamp=x["st"],
                          kslot2pos=x["ks2p"], kstamp=x["kst"], now=now)
            ls.append_token(x["new_k"], x["k8"], x["kc"], x["ctx_len"], new_kv=x["new_kv"],
                            pool=x["pool"])
        now.add_(1)

    def snapshot(layers, now):
        out = [now.clone()]
        for x in layers:
            s = x["step"]
            out += [t.clone() for t in (s.cand, s.topk, s.topk_score, s.rows, s.n_miss,
                                        s.n_key_miss, s.out.view(torch.int16), s.lse,
                                        x["hot"].view(torch.int16), x["p2s"], x["s2p"], x["st"],
                                        x["kp2s"], x["ks2p"], x["kst"], x["kcache"], x["kc"],
                                        x["ctx_len"], x["pool"].view(torch.int16))]
            out.append(x["k8"].clone())
        return out

    # the oracle's serving loop of each layer, stepped alongside copy 1 (the
    # graph's copy) from the same inputs
    shadows = [ServeShadow(wl, x["k8"], x["pool"], x["q_attn"], np_(x["ctx_len"]).tolist())
               for x in copies[1]]

    def check_with_oracle(now, what):
        for l_, (x, sh) in enumerate(zip(copies[1], shadows)):
            s = x["step"]
            tag = "%s layer %d" % (what, l_)
            sh.step(s, s.out, s.lse, x["q"].cpu(), x["w"].cpu(), now, tag)
            sh.check_state(x["hot"], (x["p2s"], x["s2p"], x["st"]),
                           (x["kp2s"], x["ks2p"], x["kst"]), x["kcache"], tag)
            sh.append(x["new_k"].cpu(), x["new_kv"].cpu())
            sh.check_stores(x["k8"], x["pool"], x["ctx_len"], tag)

    # capture on copy 1 (the capture itself runs nothing); a first eager step
    # on a side stream warms the allocator the way the capture will see it --
    # run on both copies so that they stay identical
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        token_step(copies[0], nows[0])
        token_step(copies[1], nows[1])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    check_with_oracle(1, "eager step")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        token_step(copies[1], nows[1])
    torch.cuda.synchronize()
    for k in range(4):
        token_step(copies[0], nows[0])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # every replay equals the oracle's next serving step (stamp k + 2)...
        check_with_oracle(k + 2, "replay %d" % k)
        # ...and the same step run eagerly on the identical copy
        a, b = snapshot(copies[0], nows[0]), snapshot(copies[1], nows[1])
        for i, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), (k, i)
    # the caches did get used across the steps
    assert int(copies[1][0]["step"].n_miss.sum()) < 2 * wl.topk
