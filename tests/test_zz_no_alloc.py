"""The allocation-free decode step (ls_decode_step_noalloc, on the library's
static scratch) against the step on its own workspace (ls_decode_step):
every output -- candidates, selection, scores, rows, miss counts, the hot
buffer it writes, attention output and log-sum-exp -- bit for bit, on two
calls in a row, the second with a smaller input (so the scratch holds the
first call's leftovers), then the first shape again."""
import dataclasses

import pytest
import torch

from top_sparse_attention_ls_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
BASE = synth.WORKLOADS["decode-128k-b32"]


def case(ls, wl, ctx_len, seed):
    inp = synth.indexer_inputs(wl, DEV, ctx_len=ctx_len)
    qa = synth.attention_query(wl, DEV)
    pool = synth.kv_pool(wl, DEV)
    g = torch.Generator().manual_seed(seed)
    sel = torch.stack([torch.randperm(wl.ctx, generator=g)[:wl.topk].sort().values.to(torch.int32)
                       for _ in range(wl.batch)])
    pos2slot, hot, _ = synth.hot_fill(wl, sel, pool, DEV)
    step = ls.DecodeStep(batch=wl.batch, max_ctx=wl.ctx, idx_heads=wl.idx_heads,
                         idx_dim=wl.idx_dim, n_cand=wl.n_cand, topk=wl.topk, q_heads=wl.q_heads,
                         qk_dim=wl.qk_dim, v_dim=wl.v_dim, scale=wl.scale,
                         hot_slots=wl.hot_slots, device=DEV)
    keys = inp["keys"]
    args = dict(q_idx=inp["q"], w_idx=inp["w"], kc=ls.pack_coarse(keys), k8=keys,
                ctx_len=torch.tensor(ctx_len, dtype=torch.int32, device=DEV), q_attn=qa,
                pos2slot=pos2slot, pool_kv=pool)
    return step, args, hot


def outputs(step, out, lse, hot):
    return [t.clone() for t in (step.cand, step.topk, step.topk_score, step.rows, step.n_miss,
                                out.view(torch.int16), lse, hot.view(torch.int16))]


def run_both(ls, wl, ctx_len, seed):
    step, args, hot0 = case(ls, wl, ctx_len, seed)
    hot = hot0.clone()
    out, lse = step.run(hot_kv=hot, **args)
    torch.cuda.synchronize()
    ref = outputs(step, out, lse, hot)
    for t in (step.cand, step.topk, step.rows, step.out, step.lse):
        t.fill_(-1)
    hot = hot0.clone()
    out, lse = step.run(hot_kv=hot, noalloc=True, **args)
    torch.cuda.synchronize()
    got = outputs(step, out, lse, hot)
    names = ["cand", "topk", "topk_score", "rows", "n_miss", "out", "lse", "hot"]
    for n, a, b in zip(names, ref, got):
        assert torch.equal(a, b), "%s differs from the workspace step (%s)" % (n, wl.name)


def test_noalloc_step_matches_workspace_step_twice_then_smaller(ls):
    big = dataclasses.replace(BASE, name="noalloc-big", batch=3, ctx=16384 + 5, n_cand=2048,
                              topk=512, hot_slots=1024, planted=163)
    small = dataclasses.replace(BASE, name="noalloc-small", batch=2, ctx=9000, n_cand=1024,
                                topk=256, hot_slots=300, planted=90)
    run_both(ls, big, [big.ctx, 9000, 300], seed=1)
    run_both(ls, small, [small.ctx, 4000], seed=2)
    run_both(ls, big, [big.ctx, 12000, 1], seed=3)


def test_noalloc_step_rejects_a_step_beyond_its_scratch(ls):
    # 128K x 64 needs more than the 128 MiB static scratch: refused before
    # anything is enqueued
    import ctypes
    i = ls.IdxDesc(64, 131072, 64, 128, 8192, 2048, 0, 0)
    h = ls.HotDesc(64, 131072, 2048, 4096, 576, 0)
    a = ls.AttnDesc(64, 128, 1, 576, 512, 2048, 4096 + 2048, 576, 0, 0.07, 0)
    d = ls.StepDesc(i, h, a, 1)
    rc = ls.load().ls_decode_step_noalloc(ctypes.byref(d), ctypes.byref(ls.StepIO()), None)
    assert rc == ls.LS_E_UNSUPPORTED
    assert b"static scratch" in ls.load().ls_last_error()
