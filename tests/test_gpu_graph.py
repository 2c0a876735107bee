"""The decode step captured in a HIP graph.  The step only enqueues kernels
(no allocation, no memset, no host synchronisation), so it can be captured;
every replay -- with eager steps and synchronisations in between -- must give
the eager step's results bit for bit, including the hot-buffer scratch rows
it writes and the workspace it leaves cleared for the next call."""
import dataclasses

import pytest
import torch

from top_sparse_attention_ls_amd import synth

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
