#!/usr/bin/env python3
"""Benchmark of the sparse decode step on one MI355X.

A step is one ls_decode_step call: one layer of the decode step for every
request of the batch (coarse scoring, candidate selection, refinement and
top-k, hot-buffer resolve and miss gather, split attention and combine).
Inputs are synthetic and already resident in HBM when timing starts.

Prints one JSON line (the default workload, decode-128k-b32) with:
  value       layer-steps/s (whole-step throughput, steps timed back to back)
  hbm_roofline_step  the whole step's algorithmic bytes x steps/s against the
              8 TB/s HBM peak
  roofline    the dominant kernel (coarse scoring) against the HBM peak:
              algorithmic bytes per launch / its average duration, measured
              with two HIP events the library records on the launch stream
              around that kernel, on every 8th step of the timed region
  stages_us_instrumented / stages_roofline  per-stage times from a separate
              run in which every stage is bracketed by events (each adds a
              few microseconds), and each stage's fraction of the HBM peak
  indexer_key_bytes  indexer-key bytes per step, coarse-to-fine against
              scoring every token with its full int8 key
  graph       the same steps replayed from HIP graphs (one per input replica)
  mfma_util   int8 TOPS of the coarse scoring (live events) and bf16 TFLOP/s
              of the attention kernel (instrumented run) against the dense
              MFMA peaks
  copy_GBs    a plain 1 GiB device-to-device copy, read + write bytes per
              second; read_probe: the library's read probe on the step's
              patterns (streaming read, random 1152-byte and 128-byte rows)
  cpu_baseline  the CPU oracle timed on sampled requests of the same step,
              on one thread and on up to 16 host threads at once
  io_model    (hot-buffer workloads) the measured step without its KV miss
              I/O plus the missed rows over 64 / 225 / 900 GB/s, no overlap
  key_store   (original keys on the host) PCIe bytes per step, HBM saved
  workloads   the other workloads of the same run, each with its own metric:
              tiny-4k (latency), decode-16k-b192 (pool in pinned host
              memory: PCIe-inclusive rate and achieved PCIe GB/s),
              decode-950k-b4, prefill-4k-128k (int8 TOPS, overlap, CPU
              baseline extrapolated from sampled rows)

Other workloads alone (--workload): the ones above, decode-128k-b32-hostkeys
(keys on the host behind a key cache), decode-128k-b32-serve and -serve-4l
(the serving loop: both caches committing, a token appended per step;
--graph replays each token step from a HIP graph, --microbatches splits the
batch over streams).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-decode layer-steps/s at 128K (B=32) + % of HBM roofline"
REPEATS = 5  # timed runs of K steps (the first one gives the value)
HBM_PEAK_GBS = 8000.0
STAGES = ["coarse_score", "candidate_select", "refine_topk_resolve", "miss_gather",
          "attention", "combine"]


def algorithmic_bytes(wl, n_miss_total: int, n_key_miss_total: int = 0) -> dict:
    """HBM bytes the step must move at minimum, by part (see the design
    notes).  With the original keys on the host, only the key-cache hits are
    HBM reads (plus their slot lookups); the misses cross PCIe instead."""
    B, L, H, D = wl.batch, wl.ctx, wl.idx_heads, wl.idx_dim
    row = wl.qk_dim * 2
    if wl.keys_on_host:
        refine = (B * wl.n_cand - n_key_miss_total) * D + (B * wl.n_cand * 4
                                                            if wl.key_slots else 0)
    else:
        refine = B * wl.n_cand * D
    parts = {
        "coarse_keys": B * L * D // 2,
        "refine_keys": refine,
        "slot_table": B * wl.topk * 4 if wl.hot_slots else 0,
        "miss_read": n_miss_total * row,
        "miss_write": n_miss_total * row,
        "kv_rows": (B * wl.topk * wl.kv_heads * (wl.qk_dim + wl.v_dim) * 2 if wl.attn == "mha"
                    else B * wl.topk * row),
        "attn_q": B * wl.q_heads * wl.qk_dim * 2,
        "out_lse": B * wl.q_heads * (wl.v_dim * 2 + 4),
        "idx_q_w": B * H * (D + 1),
    }
    parts["total"] = sum(parts.values())
    return parts


def load_traffic(workload):
    """Counter-measured HBM bytes per launch of the coarse kernel, if they were
    taken on the current kernel source (written by profsum from two
    rocprofv3 --pmc runs, FETCH_SIZE and WRITE_SIZE)."""
    from top_sparse_attention_ls_amd import profsum
    p = os.path.join(ROOT, "profiles", "k_coarse.%s.traffic.json" % workload)
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("kernel_sha") != profsum.coarse_kernel_sha():
        return None
    return t.get("bytes_per_launch")


def copy_bandwidth(nbytes=1 << 30, reps=5):
    """Read + write bytes per second of a plain device copy (context)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


def graph_timing(run, n_reps, steps):
    """The step captured in a HIP graph per input replica, replays timed back
    to back (the step only enqueues kernels, so it can be captured)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n_reps):
            run(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(n_reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(i)
        graphs.append(g)
    for i in range(2 * n_reps):
        graphs[i % n_reps].replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        graphs[i % n_reps].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"ms_per_step": round(ms, 5), "value": round(1000.0 / ms, 2)}


def copy_calibration(nbytes):
    """A plain device-to-device copy of known size, run only under the
    counter passes so that FETCH_SIZE / WRITE_SIZE can be scaled."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()


def read_probes(ls, wl, hot=None, keys=None, reps=5):
    """Bandwidth the hardware delivers to the step's read patterns (the
    library's ls_read_probe, timed with events): a streaming read of 1 GiB,
    and gathers of random whole rows drawn request by request as the step
    draws them -- the step's number of 1152-byte latent rows from each
    request's hot-buffer block (the attention's pattern), and its number of
    128-byte key rows from each request's key block (the refinement's).
    Context for the roofline figures."""
    import torch
    dev = torch.device("cuda:0")
    out = {}
    # 1 GiB, four times the 256 MB Infinity Cache: reading it evicts what an
    # earlier probe left there, so every timed probe reads HBM, as the step does
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)

    def timed(fn):
        fn()
        total = 0.0
        for _ in range(reps):
            ls.read_probe(buf)   # evict (untimed)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1)
        return total / reps * 1e-3

    t = timed(lambda: ls.read_probe(buf))
    out["seq_read_GBs"] = round((1 << 30) / t / 1e9, 1)
    g = torch.Generator(device=dev).manual_seed(5)

    def per_request(n_req, block, n_each):
        r = torch.randint(0, block, (n_req, n_each), generator=g, device=dev, dtype=torch.int64)
        r += torch.arange(n_req, device=dev, dtype=torch.int64)[:, None] * block
        return r.to(torch.int32).flatten()

    if hot is not None:
        B, block = hot.shape[0], hot.shape[1]
        rows = per_request(B, block, wl.topk)
        t = timed(lambda: ls.read_probe(hot, rows, 1152))
        out["rows_1152B_GBs"] = round(rows.numel() * 1152 / t / 1e9, 1)
        out["rows_1152B"] = "%d random rows of each request's %d-row hot-buffer block" % (
            wl.topk, block)
    if keys is not None:
        B, block = keys.shape[0], keys.shape[1]
        rows = per_request(B, block, wl.n_cand)
        t = timed(lambda: ls.read_probe(keys, rows, 128))
        out["rows_128B_GBs"] = round(rows.numel() * 128 / t / 1e9, 1)
        out["rows_128B"] = "%d random rows of each request's %d-row key block" % (wl.n_cand,
                                                                                   block)
    out["note"] = ("each timed probe follows an untimed read of 1 GiB (Infinity Cache evicted) "
                   "and is bracketed by its own event pair (a few microseconds of overhead)")
    del buf
    torch.cuda.empty_cache()
    return out


def metric_for(wl) -> str:
    """The metric string of a decode workload's line (the headline workload
    keeps the benchmark's own metric)."""
    if wl.name == "decode-128k-b32":
        return METRIC
    ctx = "%dK" % (wl.ctx // 1024) if wl.ctx % 1024 == 0 else "%dK" % round(wl.ctx / 1000)
    extra = ""
    if wl.attn == "mha":
        extra = ", MHA %dx%d, latency" % (wl.q_heads, wl.qk_dim)
    if wl.pool_on_host:
        extra += ", pool in pinned host memory (PCIe-inclusive)"
    if wl.keys_on_host:
        extra += ", original keys in pinned host memory"
    return "sparse-decode layer-steps/s at %s (B=%d)%s + %% of HBM roofline" % (ctx, wl.batch,
                                                                                extra)


def indexer_key_bytes(wl, ab) -> dict:
    """Indexer-key bytes read per step: the coarse-to-fine pass (every compact
    key, plus the candidates' original keys) against scoring every token
    with its full int8 key."""
    full = wl.batch * wl.ctx * wl.idx_dim
    c2f = ab["coarse_keys"] + ab["refine_keys"]
    return {"coarse_pass": ab["coarse_keys"], "refine": ab["refine_keys"],
            "coarse_to_fine_total": c2f, "full_key_scoring": full,
            "ratio": round(c2f / full, 4)}


def build_inputs(ls, synth, wl, dev, replicas):
    import torch
    inp = synth.indexer_inputs(wl, dev)
    keys = inp["keys"]
    kc = ls.pack_coarse(keys)
    q_attn = synth.attention_query(wl, dev)
    ctx_len = torch.full((wl.batch,), wl.ctx, dtype=torch.int32, device=dev)
    pool = pos2slot = hot = kv = None
    n_miss = [0] * wl.batch
    if wl.hot_slots:
        pool = synth.kv_pool(wl, dev, pin=wl.pool_on_host, gen_device=dev)
        # the hot buffer is laid out from this workload's own selection,
        # computed once here (setup, untimed) so that exactly the stated share
        # misses
        cand = ls.index_coarse(inp["q"], inp["w"], kc, ctx_len, wl.n_cand)
        sel, _ = ls.refine_topk(inp["q"], inp["w"], keys, cand, ctx_len, wl.topk)
        pos2slot, hot, n_miss = synth.hot_fill(wl, sel, pool, dev)
    else:
        kv = synth.kv_cache_mha(wl, dev)
    key_cache, n_key_miss = None, None
    if wl.key_slots:
        # the indexer-key cache is laid out from the same candidate set
        kp, kcache, n_key_miss = synth.key_cache_fill(wl, cand, keys, dev)
        key_cache = dict(kpos2slot=kp, kcache=kcache)
    if wl.keys_on_host:
        # the original keys leave HBM: one pinned host copy, shared by the
        # replicas (as a host pool is)
        keys = keys.to("cpu").pin_memory()
    reps = []
    for r in range(replicas):
        def rep(t):
            return t if (r == 0 or t is None) else t.clone()
        rep_ = dict(q_idx=inp["q"], w_idx=inp["w"], ctx_len=ctx_len,
                    k8=keys if wl.keys_on_host else rep(keys), kc=rep(kc),
                    q_attn=rep(q_attn), pos2slot=rep(pos2slot), hot_kv=rep(hot), pool_kv=pool)
        if kv is not None:
            rep_.update(k_cache=rep(kv[0]), v_cache=rep(kv[1]))
        if key_cache is not None:
            rep_.update({k: rep(v) for k, v in key_cache.items()})
        reps.append(rep_)
    torch.cuda.synchronize()
    return dict(reps=reps, n_miss=n_miss, n_key_miss=n_key_miss, inp=inp, q_attn=q_attn,
                pool=pool, pos2slot=pos2slot, hot=hot, kv=kv)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_threads() -> int:
    """Host threads of the parallel CPU baseline: the CPU share of one GPU
    (16), or fewer if the machine has fewer."""
    return max(1, min(16, os.cpu_count() or 1))


def timed_pool(fn, items, n_threads):
    """fn over items on n_threads host threads; (wall seconds, per-item
    seconds).  The oracle's C calls release the interpreter lock."""
    import concurrent.futures

    def one(x):
        t0 = time.perf_counter()
        fn(x)
        return time.perf_counter() - t0

    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(n_threads) as ex:
        per = list(ex.map(one, items))
    return time.perf_counter() - t0, per


def cpu_baseline(wl, st, n_single, n_parallel):
    """The oracle, as it stands, on sampled requests of the same step: one
    thread on n_single requests, then n_parallel requests at once on that
    many host threads (independent requests, as independent processes would
    split the batch).  value = the parallel rate scaled to the batch."""
    import numpy as np
    import torch
    from oracle import oracle as orc

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    inp = st["inp"]

    def prepared(b):
        x = dict(q=inp["q"][b].cpu().numpy(), w=inp["w"][b].cpu().numpy(),
                 keys=inp["keys"][b].cpu().numpy(), qa=bits(st["q_attn"][b]))
        if wl.hot_slots:
            x.update(p2s=st["pos2slot"][b].cpu().numpy(), hot=bits(st["hot"][b]).copy(),
                     pool=bits(st["pool"][b]))
        else:
            x.update(kc=bits(st["kv"][0][b]).reshape(-1), vc=bits(st["kv"][1][b]).reshape(-1))
        return x

    def run(x):
        if wl.hot_slots:
            orc.decode_request(x["q"], x["w"], x["keys"], wl.ctx, wl.n_cand, wl.topk, x["qa"],
                               wl.scale, pos2slot=x["p2s"], hot_bits=x["hot"],
                               pool_bits=x["pool"], v_dim=wl.v_dim, row_stride=wl.qk_dim)
        else:
            orc.decode_request(x["q"], x["w"], x["keys"], wl.ctx, wl.n_cand, wl.topk, x["qa"],
                               wl.scale, k_cache_bits=x["kc"], v_cache_bits=x["vc"],
                               n_kv_heads=wl.kv_heads, v_dim=wl.v_dim,
                               row_stride=wl.kv_heads * wl.qk_dim, head_stride=wl.qk_dim)

    res = {"unit": "layer-steps/s", "kind": "oracle", "cpu_model": cpu_model(),
           "host_cpus_visible": os.cpu_count()}
    per_single = None
    if n_single > 0:
        xs = [prepared(b % wl.batch) for b in range(n_single)]
        _, per = timed_pool(run, xs, 1)
        per_single = sum(per) / len(per)
        del xs
        res["single_thread"] = {"value": 1.0 / (per_single * wl.batch), "cores": 1,
                                "s_per_request": round(per_single, 3),
                                "requests_sampled": n_single}
    P = min(n_parallel, host_threads())
    if P > 0:
        xs = [prepared(b % wl.batch) for b in range(P)]
        wall, per = timed_pool(run, xs, P)
        del xs
        rate = P / wall / wl.batch
        res.update(value=rate, cores=P,
                   sample="%d requests of %s at once on %d host threads (whole step per "
                          "request: coarse scores, candidates, refine, top-k, hot resolve + "
                          "gather, attention; single-threaded C each), %.2f s wall, scaled to "
                          "the %d-request batch" % (P, wl.name, P, wall, wl.batch))
        if per_single is None:
            res["single_thread"] = {"value": 1.0 / (sum(per) / P * wl.batch), "cores": 1,
                                    "s_per_request": round(sum(per) / P, 3),
                                    "note": "per-request times inside the parallel run"}
    else:
        res.update(value=res["single_thread"]["value"], cores=1,
                   sample="%d requests of %s, single-threaded C" % (n_single, wl.name))
    return res


STAGE_KERNELS = {
    "coarse_score": "k_coarse32 (k_coarse up to 16 heads)",
    "candidate_select": "k_topc_filter + k_topc_emit",
    "refine_topk_resolve": "k_refine + k_topk_hist",
    "miss_gather": "k_hot_gather",
    "attention": "k_attn_mfma",
    "combine": "k_combine (k_combine_wide when the rows are few)",
}


def gather_folded(wl) -> bool:
    """Whether the library folds the miss gather into the attention kernel's
    tile DMA for this workload (hot buffer, pool in device memory, latent
    rows on the MFMA path)."""
    return bool(wl.hot_slots) and not wl.pool_on_host and wl.kv_heads in (0, 1) and \
        wl.qk_dim == 576 and wl.v_dim == 512 and wl.q_heads % 16 == 0 and wl.q_heads <= 128


def stage_bytes(wl, ab) -> dict:
    """Algorithmic bytes of each stage (the parts of algorithmic_bytes)."""
    return {
        "coarse_score": ab["coarse_keys"] + ab["idx_q_w"],
        "candidate_select": 0,
        "refine_topk_resolve": ab["refine_keys"] + ab["slot_table"],
        "miss_gather": ab["miss_read"] + ab["miss_write"],
        "attention": ab["kv_rows"] + ab["attn_q"],
        "combine": ab["out_lse"],
    }


def run_decode(ls, synth, wl, steps, warmup, replicas, full=True, n_single=0, n_parallel=0,
               with_graph=None):
    """Time K = steps whole decode steps of workload wl back to back (after
    warmup untimed ones) and return the result object.  full: also the
    repeats, the HIP-graph replay and the stage breakdown of an instrumented
    run; otherwise only the timed run and a short instrumented run.
    with_graph: time the HIP-graph replay too (default: when full)."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] building inputs for %s" % wl.name, file=sys.stderr, flush=True)
    st = build_inputs(ls, synth, wl, dev, replicas)
    reps, n_miss, n_key_miss = st["reps"], st["n_miss"], st["n_key_miss"]
    mha = not wl.hot_slots
    step = ls.DecodeStep(batch=wl.batch, max_ctx=wl.ctx, idx_heads=wl.idx_heads,
                         idx_dim=wl.idx_dim, n_cand=wl.n_cand, topk=wl.topk,
                         q_heads=wl.q_heads, qk_dim=wl.qk_dim, v_dim=wl.v_dim, scale=wl.scale,
                         hot_slots=wl.hot_slots, pool_on_host=wl.pool_on_host,
                         keys_on_host=wl.keys_on_host, key_slots=wl.key_slots,
                         kv_heads=wl.kv_heads,
                         kv_row_stride=wl.kv_heads * wl.qk_dim if mha else None,
                         kv_head_stride=wl.qk_dim if mha else 0, device=dev)

    def run(i, events=None):
        r = reps[i % len(reps)]
        step.run(q_idx=r["q_idx"], w_idx=r["w_idx"], kc=r["kc"], k8=r["k8"],
                 ctx_len=r["ctx_len"], q_attn=r["q_attn"], pos2slot=r["pos2slot"],
                 hot_kv=r["hot_kv"], pool_kv=r["pool_kv"], kpos2slot=r.get("kpos2slot"),
                 kcache=r.get("kcache"), k_cache=r.get("k_cache"), v_cache=r.get("v_cache"),
                 events=events)

    # host-side set-up first (the miss-count check after one step, the
    # events), so that the warm-up runs right up to the timed region and the
    # GPU enters it busy rather than after a host-side pause
    run(0)
    torch.cuda.synchronize()
    if wl.hot_slots:
        miss_now = step.n_miss.cpu().tolist()
        assert miss_now == n_miss, "hot buffer miss counts drifted: %s" % miss_now
    if wl.keys_on_host:
        # candidates whose key is not in the key cache: their rows cross PCIe
        c = step.cand.long()
        kp = reps[0].get("kpos2slot")
        if kp is None:
            key_miss_now = (c >= 0).sum(1).tolist()
        else:
            hit = kp.gather(1, c.clamp(min=0)) >= 0
            key_miss_now = ((c >= 0) & ~hit).sum(1).tolist()
        if n_key_miss is not None:
            assert key_miss_now == n_key_miss, "key cache miss counts drifted"
        n_key_miss = key_miss_now

    K = steps
    # timed region: whole steps back to back; on every SAMPLE-th step the
    # library also records two events around the coarse kernel (an event
    # costs the stream a few microseconds, so only the measured kernel is
    # bracketed, and only on a sample of the steps)
    SAMPLE = 8
    coarse_ev = {}
    for i in range(0, K, SAMPLE):
        coarse_ev[i] = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for pair in coarse_ev.values():  # create the underlying events before use
        for e in pair:
            e.record()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record()
    t_end.record()
    print("[bench] %s: warmup %d, then timing %d steps" % (wl.name, warmup, K), file=sys.stderr,
          flush=True)
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(K):
        pair = coarse_ev.get(i)
        run(i, None if pair is None else [pair[0], pair[1]] + [None] * (ls.STEP_EVENTS - 2))
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K
    coarse_ms = sum(p[0].elapsed_time(p[1]) for p in coarse_ev.values()) / len(coarse_ev)

    # the same K steps timed again, without any event inside: the spread of
    # the rate over repeated runs (the value above is the first run's)
    rep_ms = [ms_per_step]
    for _ in range(REPEATS - 1 if full else 0):
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        r0.record()
        for i in range(K):
            run(i)
        r1.record()
        torch.cuda.synchronize()
        rep_ms.append(r0.elapsed_time(r1) / K)
    rates = sorted(1000.0 / m for m in rep_ms)

    # stage breakdown from a separate instrumented run (every stage bracketed)
    n_inst = min(K, 20 if full else 8)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ls.STEP_EVENTS)]
           for _ in range(n_inst)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(n_inst):
        run(i, evs[i])
    torch.cuda.synchronize()
    stage_ms = [0.0] * (ls.STEP_EVENTS - 1)
    for row in evs:
        for s_ in range(ls.STEP_EVENTS - 1):
            stage_ms[s_] += row[s_].elapsed_time(row[s_ + 1]) / n_inst

    graph = None
    if full if with_graph is None else with_graph:
        # the same steps replayed from HIP graphs (reported beside the eager value)
        try:
            graph = graph_timing(run, len(reps), K)
        except Exception as exc:  # reported, never hidden: the eager value stands
            graph = {"error": repr(exc)}
        torch.cuda.synchronize()

    ab = algorithmic_bytes(wl, sum(n_miss), sum(n_key_miss or [0]))
    steps_per_s = 1000.0 / ms_per_step
    coarse_bytes = ab["coarse_keys"] + ab["idx_q_w"]
    achieved = coarse_bytes / (coarse_ms * 1e-3) / 1e9
    step_frac = ab["total"] * steps_per_s / 1e9 / HBM_PEAK_GBS
    result = {
        "metric": metric_for(wl),
        "value": round(steps_per_s, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.batch, "ctx": wl.ctx, "idx_heads": wl.idx_heads,
            "idx_dim": wl.idx_dim, "n_cand": wl.n_cand, "topk": wl.topk,
            "attention": "%s %d heads x %d" % (wl.attn.upper(), wl.q_heads, wl.qk_dim),
            "v_dim": wl.v_dim, "hot_slots": wl.hot_slots, "miss_rate": wl.miss_rate,
            "pool": ("pinned-host" if wl.pool_on_host else "hbm") if wl.hot_slots else "none",
            "keys": "pinned-host" if wl.keys_on_host else "hbm",
            "key_slots": wl.key_slots, "key_miss_rate": wl.key_miss_rate,
            "replicas": replicas, "parallelism": "single-gpu",
        },
        "hbm_roofline_step": {
            "algorithmic_bytes": ab["total"],
            "achieved_GBs": round(ab["total"] * steps_per_s / 1e9, 1),
            "frac": round(step_frac, 4),
        },
        # the dominant kernel of the step against the HBM peak (live events);
        # the whole step's fraction is hbm_roofline_step.frac
        "roofline": {
            "kernel": "coarse_score (k_coarse32)",
            "scope": "dominant kernel; whole step in hbm_roofline_step",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(wl.name),
            "algorithmic_bytes_per_launch": coarse_bytes,
            "avg_launch_us": round(coarse_ms * 1000, 2),
            "step_frac": round(step_frac, 4),
        },
        "coarse_events_sampled": len(coarse_ev),
        "stages_us_instrumented": {n: round(v * 1000, 2) for n, v in zip(STAGES, stage_ms)},
        "request_layer_steps_per_s": round(steps_per_s * wl.batch, 1),
        "indexer_key_bytes": indexer_key_bytes(wl, ab),
    }
    # every stage against its own roofline (stage times from the instrumented
    # run: each includes the event it ends on, a few microseconds)
    sb = stage_bytes(wl, ab)
    stage_us = {n: v * 1000 for n, v in zip(STAGES, stage_ms)}
    kernels = dict(STAGE_KERNELS)
    if gather_folded(wl):
        # the library folds the miss gather into the attention's tile DMA
        # (pool in HBM, latent rows): no kernel runs between the two events,
        # so the gather's bytes and the gap's microseconds (event overhead)
        # belong to the attention stage
        stage_us["attention"] += stage_us["miss_gather"]
        stage_us["miss_gather"] = 0.0
        sb["attention"] += sb["miss_gather"]
        sb["miss_gather"] = 0
        kernels["miss_gather"] = "folded into k_attn_mfma (tile DMA)"
        kernels["attention"] = "k_attn_mfma (with the miss gather)"
    result["stages_roofline"] = {
        n: {"kernels": kernels[n], "us": round(stage_us[n], 2), "algorithmic_bytes": sb[n],
            "frac_of_hbm": round(sb[n] / (stage_us[n] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            if stage_us[n] > 0 else None}
        for n in STAGES}
    if mha:
        result["latency_us"] = round(ms_per_step * 1000, 2)
        result["hbm_roofline_step"]["note"] = ("%.2f MB per step stays in the caches: the step "
                                               "is latency-bound" % (ab["total"] / 1e6))
    if full:
        result["repeats"] = {
            "runs": len(rates), "steps_each": K,
            "median": round(rates[len(rates) // 2], 2),
            "p10": round(rates[max(0, int(0.1 * (len(rates) - 1)))], 2),
            "p90": round(rates[int(round(0.9 * (len(rates) - 1)))], 2),
            "note": "layer-steps/s of the first run (the value) and of the same K steps "
                    "repeated without events",
        }
    if graph is not None:
        result["graph"] = graph
    if wl.keys_on_host:
        full_keys = wl.batch * wl.ctx * wl.idx_dim
        cache = wl.batch * wl.key_slots * (wl.idx_dim) + (wl.batch * wl.ctx * 4
                                                           if wl.key_slots else 0)
        pcie = sum(n_key_miss) * wl.idx_dim
        result["key_store"] = {
            "pcie_key_bytes_per_step": pcie,
            "pcie_GBs_at_value": round(pcie * steps_per_s / 1e9, 2),
            "hbm_bytes_full_keys": full_keys,
            "hbm_bytes_key_cache_and_table": cache,
            "hbm_saved_bytes": full_keys - cache,
            "hbm_saved_per_request": (full_keys - cache) // wl.batch,
        }
    if wl.hot_slots:
        # the compute-plus-I/O model of the hot-buffer analysis: the measured
        # step without its KV miss I/O, plus the missed rows' bytes over a
        # link of each modelled bandwidth, the two not overlapping
        stage = dict(zip(STAGES, stage_ms))
        folded = gather_folded(wl)
        compute_us = (sum(stage_ms) - (0.0 if folded else stage["miss_gather"])) * 1000
        miss_bytes = sum(n_miss) * wl.qk_dim * 2
        result["io_model"] = {
            "compute_us_without_kv_io": round(compute_us, 1),
            "kv_miss_bytes": miss_bytes,
            "modeled_us": {str(bw): round(compute_us + miss_bytes / (bw * 1e3), 1)
                           for bw in (64, 225, 900)},
            "measured_us": round(ms_per_step * 1000, 1),
            "measured_gather_us": None if folded else round(stage["miss_gather"] * 1000, 1),
            "gather_GBs": None if folded else round(
                miss_bytes / (stage["miss_gather"] * 1e-3) / 1e9, 1),
            "link": "pinned host (PCIe)" if wl.pool_on_host else "HBM",
            "note": ("stage times from the instrumented run (an event between stages)" +
                     ("; the gather is folded into the attention's tile DMA, so its time is "
                      "not separable and the compute figure includes it" if folded else "")),
        }
        if wl.pool_on_host:
            result["pcie"] = {
                "miss_bytes_per_step": miss_bytes,
                "gather_us": round(stage["miss_gather"] * 1000, 1),
                "achieved_GBs": round(miss_bytes / (stage["miss_gather"] * 1e-3) / 1e9, 1),
                "rate_without_pcie_gather": round(1e6 / compute_us, 1),
                "note": "value is PCIe-inclusive (the gather reads the missed rows over PCIe "
                        "inside the step); the HBM fraction counts only device bytes",
            }
    coarse_ops = 2 * wl.batch * wl.ctx * wl.idx_heads * wl.idx_dim
    attn_flops = 2 * wl.batch * wl.q_heads * wl.topk * (wl.qk_dim + wl.v_dim)
    attn_ms = stage_ms[STAGES.index("attention")]
    result["mfma_util"] = {
        "coarse_int8_TOPS": round(coarse_ops / (coarse_ms * 1e-3) / 1e12, 1),
        "coarse_frac_of_5000": round(coarse_ops / (coarse_ms * 1e-3) / 1e12 / 5000.0, 4),
        "attention_bf16_TFLOPs": round(attn_flops / (attn_ms * 1e-3) / 1e12, 1),
        "attention_frac_of_2500": round(attn_flops / (attn_ms * 1e-3) / 1e12 / 2500.0, 4),
        "note": "from event timings; the counter-measured busy fractions are in profiles/",
    }
    if n_single > 0 or n_parallel > 0:
        print("[bench] %s: cpu baseline" % wl.name, file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, st, n_single, n_parallel)
    probe_src = (st["hot"] if wl.hot_slots else None,
                 st["inp"]["keys"] if not wl.keys_on_host else None)
    del reps, st, step
    return result, probe_src


def run_prefill(ls, synth, wl, steps, warmup, n_rows_cpu=0):
    """The prefill-chunk indexer: every layer's history streamed from pinned
    host memory through two device buffers, the copy of layer l+1 overlapping
    the indexer of layer l.  value = int8 TOPS of the causal score GEMM over
    the whole streamed run; also the compute-only time (keys already on the
    device) and the overlap efficiency (compute-only / streamed).  With
    n_rows_cpu > 0 the oracle is timed on that many sampled query rows of
    layer 0 on as many host threads, and its rate extrapolated to the chunk."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Tq, L, H, D, K = wl.n_query, wl.ctx, wl.idx_heads, wl.idx_dim, wl.topk
    q_pos0 = L - Tq
    print("[bench] building %d prefill layers" % wl.layers, file=sys.stderr, flush=True)
    layers = [synth.prefill_inputs(wl, l, dev) for l in range(wl.layers)]
    qs = [x["q"] for x in layers]
    ws_ = [x["w"] for x in layers]
    kh = [x["keys"].cpu().pin_memory() for x in layers]
    kd = [x["keys"] for x in layers]
    buf0 = torch.empty((L, D), dtype=torch.int8, device=dev)
    buf1 = torch.empty((L, D), dtype=torch.int8, device=dev)
    copy_stream = torch.cuda.Stream(device=dev)
    pairs = sum(min(q_pos0 + i + 1, L) for i in range(Tq))   # causal query-key pairs
    ops = 2 * pairs * H * D * wl.layers

    def streamed():
        return ls.prefill_stream_layers(qs, ws_, kh, q_pos0, K, buf0, buf1, copy_stream)

    def compute_only():
        return [ls.prefill_index_topk(qs[l], ws_[l], kd[l], q_pos0, K) for l in range(wl.layers)]

    for _ in range(max(warmup, 1)):
        streamed()
        compute_only()
    torch.cuda.synchronize()
    steps = max(1, min(steps, 10))

    def timed(fn):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    print("[bench] timing %d streamed chunks" % steps, file=sys.stderr, flush=True)
    ms_stream = timed(streamed)
    ms_compute = timed(compute_only)
    tops = ops / (ms_stream * 1e-3) / 1e12
    tops_c = ops / (ms_compute * 1e-3) / 1e12
    result = {
        "metric": "prefill-chunk indexer int8 TOPS (%d layers streamed)" % wl.layers,
        "value": round(tops, 1),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": max(warmup, 1),
        "ms_per_step": round(ms_stream, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "n_query": Tq, "ctx": L, "idx_heads": H, "idx_dim": D,
                   "topk": K, "layers": wl.layers, "keys": "pinned-host, 2 device buffers",
                   "parallelism": "single-gpu"},
        "roofline": {"kernel": "whole indexer (scores + selection)", "bound": "mfma",
                     "achieved": round(tops, 1), "peak": 5000.0, "unit": "TOPS",
                     "frac": round(tops / 5000.0, 4), "traffic": None},
        "compute_only_ms": round(ms_compute, 4),
        "compute_only_tops": round(tops_c, 1),
        "overlap_efficiency": round(ms_compute / ms_stream, 4),
        "h2d_bytes_per_layer": L * D,
        "int8_ops": ops,
    }
    if n_rows_cpu > 0:
        import numpy as np
        from oracle import oracle as orc
        P = min(n_rows_cpu, host_threads())
        rows = np.linspace(0, Tq - 1, n_rows_cpu).round().astype(int).tolist()
        q0, w0, k0 = qs[0].cpu().numpy(), ws_[0].cpu().numpy(), kh[0].numpy()
        print("[bench] prefill cpu baseline on %d rows" % len(rows), file=sys.stderr, flush=True)
        wall, per = timed_pool(lambda i: orc.prefill_row(q0[i], w0[i], k0, q_pos0 + i, K), rows,
                               P)
        row_ops = sum(2 * (q_pos0 + i + 1) * H * D for i in rows)
        # each row's time scales with the keys it sees; extrapolate by ops
        rate = row_ops / wall
        result["cpu_baseline"] = {
            "value": round(rate / 1e12, 6), "unit": "TOPS", "cores": P, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus_visible": os.cpu_count(),
            "extrapolated_ms_per_chunk": round(ops / rate * 1e3, 1),
            "single_thread_s_per_row": round(sum(per) / len(per), 3),
            "sample": "%d query rows of layer 0 (first, last, evenly spaced) on %d host "
                      "threads, single-threaded C each (%.2f s wall); extrapolated to the "
                      "%d x %d-layer chunk by int8 operations" % (len(rows), P, wall, Tq,
                                                                 wl.layers),
        }
    del layers, qs, ws_, kh, kd, buf0, buf1
    return result


def micro_batch(ls, st, b0, Bm, wl, dev):
    """Requests [b0, b0 + Bm) of a layer's serving state: views of every
    per-request tensor (the batch is the leading dimension, so each view is
    contiguous) and a step of their own."""
    sl = slice(b0, b0 + Bm)
    y = {k: v[sl] for k, v in st.items() if k not in ("qs", "new_k", "new_kv")}
    y["qs"] = [q[sl] for q in st["qs"]]
    y["new_k"] = [t[sl] for t in st["new_k"]]
    y["new_kv"] = [t[sl] for t in st["new_kv"]]
    y["step"] = ls.DecodeStep(batch=Bm, max_ctx=wl.ctx, idx_heads=wl.idx_heads,
                              idx_dim=wl.idx_dim, n_cand=wl.n_cand, topk=wl.topk,
                              q_heads=wl.q_heads, qk_dim=wl.qk_dim, v_dim=wl.v_dim,
                              scale=wl.scale, hot_slots=wl.hot_slots, keys_on_host=True,
                              key_slots=wl.key_slots, commit_hot=True, commit_keys=True,
                              device=dev)
    return y


def run_serve(ls, synth, wl, args):
    """Decode steps in a row as in serving, over wl.layers layers (default
    one): per layer, the original keys in pinned host memory behind the
    indexer-key cache, both caches starting empty and committing every step
    (least recently used), one new token appended per step and request; the
    indexer queries drift from step to step (a ring of 32 drifted queries per
    layer).  One token step runs every layer in turn, then advances the
    stamp counter on the device.  value = layer-steps/s of that loop; with
    --graph the whole token step (every layer, its commits and appends, the
    counter) is captured once in a HIP graph and replayed, one graph per
    query of the ring.  The PCIe bytes are the key rows of the candidates
    missing the key cache."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, L, H, D, C, K = wl.batch, wl.ctx, wl.idx_heads, wl.idx_dim, wl.n_cand, wl.topk
    S, SK, row = wl.hot_slots, wl.key_slots, wl.qk_dim
    n_layers = max(wl.layers, 1)
    mb = args.microbatches or wl.serve_microbatches
    if B % mb:
        raise SystemExit("the batch of %d does not split into %d micro-batches" % (B, mb))
    if mb > 1 and args.graph:
        raise SystemExit("--graph replays one stream: use it with one micro-batch")
    Bm = B // mb
    ring, n_stat = 32, 8
    total = args.warmup + args.steps + n_stat + 2 * ring
    print("[bench] building serving state for %s (%d layers)" % (wl.name, n_layers),
          file=sys.stderr, flush=True)
    layers = []
    for layer in range(n_layers):
        lw = dataclasses.replace(wl, seed=wl.seed + 7919 * layer)
        inp = synth.indexer_inputs(lw, dev)
        kc = ls.pack_coarse(inp["keys"])
        k8 = inp["keys"].to("cpu").pin_memory()
        del inp["keys"]
        g = synth.generator(lw.seed, 100, 0, dev)
        qs = [inp["q"]]
        for _ in range(ring - 1):
            qs.append(synth.drift_query(qs[-1], wl.serve_drift, g, dev))
        st = dict(
            w=inp["w"], qs=qs, kc=kc, k8=k8, pool=synth.kv_pool(lw, dev, gen_device=dev),
            q_attn=synth.attention_query(lw, dev),
            ctx_len=torch.full((B,), L - total - 1, dtype=torch.int32, device=dev),
            new_k=[synth.int8_normal((B, D), 24.0, g, dev) for _ in range(4)],
            new_kv=[synth.bf16_normal((B, row), g, dev) for _ in range(4)],
            hot=torch.zeros((B, S + K, row), dtype=torch.bfloat16, device=dev),
            p2s=torch.full((B, L), -1, dtype=torch.int32, device=dev),
            s2p=torch.full((B, S), -1, dtype=torch.int32, device=dev),
            st=torch.zeros((B, S), dtype=torch.int32, device=dev),
            kp2s=torch.full((B, L), -1, dtype=torch.int32, device=dev),
            ks2p=torch.full((B, SK), -1, dtype=torch.int32, device=dev),
            kst=torch.zeros((B, SK), dtype=torch.int32, device=dev),
            kcache=torch.zeros((B, SK, D), dtype=torch.int8, device=dev))
        # micro-batches: contiguous request ranges (views), each its own step
        st["mb"] = [micro_batch(ls, st, m * Bm, Bm, wl, dev) for m in range(mb)]
        layers.append(st)
    now = torch.ones((1,), dtype=torch.int32, device=dev)
    side_streams = [torch.cuda.Stream() for _ in range(mb - 1)]
    sel_ev = [[torch.cuda.Event() for _ in range(mb)] for _ in layers]

    def token_step(i):
        # micro-batch m runs on stream m and starts each layer once micro-batch
        # m-1 has selected its candidates, so that one's key reads over PCIe
        # overlap the next one's coarse pass in HBM
        main = torch.cuda.current_stream()
        streams = [main] + side_streams
        for strm in side_streams:
            strm.wait_stream(main)
        for li, x in enumerate(layers):
            for m, y in enumerate(x["mb"]):
                with torch.cuda.stream(streams[m]):
                    if m > 0:
                        streams[m].wait_event(sel_ev[li][m - 1])
                    ev = None
                    if m < mb - 1:
                        ev = [None] * ls.STEP_EVENTS
                        ev[2] = sel_ev[li][m]
                    y["step"].run(q_idx=y["qs"][i % ring], w_idx=y["w"], kc=y["kc"], k8=y["k8"],
                                  ctx_len=y["ctx_len"], q_attn=y["q_attn"], pos2slot=y["p2s"],
                                  hot_kv=y["hot"], pool_kv=y["pool"], kpos2slot=y["kp2s"],
                                  kcache=y["kcache"], slot2pos=y["s2p"], stamp=y["st"],
                                  kslot2pos=y["ks2p"], kstamp=y["kst"], now=now, events=ev)
                    ls.append_token(y["new_k"][i % 4], y["k8"], y["kc"], y["ctx_len"],
                                    new_kv=y["new_kv"][i % 4], pool=y["pool"])
        for strm in side_streams:
            main.wait_stream(strm)
        now.add_(1)

    counter = [0]
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(ring):       # warm the caches (and the allocator) eagerly
                token_step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for i in range(ring):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                token_step(i)
            graphs.append(gr)
        torch.cuda.synchronize()

        def one():
            graphs[counter[0] % ring].replay()
            counter[0] += 1
    else:
        def one():
            token_step(counter[0])
            counter[0] += 1

    torch.cuda.synchronize()
    print("[bench] warmup %d, then timing %d token steps" % (args.warmup, args.steps),
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        one()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps / n_layers       # per layer-step
    hot_miss, key_miss = [], []
    for _ in range(n_stat):
        one()
        torch.cuda.synchronize()
        hot_miss.append(sum(int(y["step"].n_miss.sum()) for x in layers for y in x["mb"])
                        / n_layers)
        key_miss.append(sum(int(y["step"].n_key_miss.sum()) for x in layers for y in x["mb"])
                        / n_layers)
    km = sum(key_miss) / n_stat
    result = {
        "metric": "sparse-decode layer-steps/s, serving loop (commits + append)",
        "value": round(1000.0 / ms, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "ctx": L, "idx_heads": H, "idx_dim": D,
                   "n_cand": C, "topk": K, "hot_slots": S, "key_slots": SK, "layers": n_layers,
                   "query_drift": wl.serve_drift, "keys": "pinned-host", "pool": "hbm",
                   "launch": "hip-graph per token step" if args.graph else "eager",
                   "micro_batches": mb,
                   "parallelism": "single-gpu"},
        "token_steps_per_s": round(1000.0 / (ms * n_layers), 2),
        # per layer: the original keys leave HBM; the key cache, its slot
        # table and its LRU state (slot -> token, stamp) stay
        "memory_per_layer": {
            "hbm_bytes_full_keys": B * L * D,
            "hbm_bytes_key_cache_and_tables": B * SK * D + B * L * 4 + B * SK * 8,
            "hbm_saved_bytes": B * L * D - (B * SK * D + B * L * 4 + B * SK * 8),
        },
        "emergent": {
            "hot_miss_rate": round(sum(hot_miss) / n_stat / (B * K), 4),
            "key_miss_rate": round(km / (B * C), 4),
            "pcie_key_bytes_per_layer_step": int(km * D),
            "pcie_GBs_at_value": round(km * D * 1000.0 / ms / 1e9, 2),
            "steps_sampled": n_stat,
        },
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=60,
                    help="untimed steps first (the GPU reaches its steady clocks)")
    ap.add_argument("--workload", default="decode-128k-b32")
    ap.add_argument("--replicas", type=int, default=2)
    ap.add_argument("--cpu-sample", type=int, default=16,
                    help="requests the CPU oracle baseline runs at once on as many host threads "
                         "(prefill: four times as many query rows; 0 = skip the baseline)")
    ap.add_argument("--extras", type=int, default=1,
                    help="default workload: also measure the other workloads (4K latency, "
                         "16K x 192 with the pool on the host, 950K x 4, the prefill chunk) "
                         "and report them under 'workloads' (0 = skip)")
    ap.add_argument("--microbatches", type=int, default=0,
                    help="serving workloads: split the batch into this many micro-batches on "
                         "their own streams (0: the workload's default)")
    ap.add_argument("--graph", action="store_true",
                    help="serving workloads: replay each token step from a HIP graph")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="MiB of a plain device copy run after timing (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import gc
    import torch
    import top_sparse_attention_ls_amd as ls
    from top_sparse_attention_ls_amd import synth

    ls.load()
    wl = synth.WORKLOADS[args.workload]
    if wl.n_query:
        print(json.dumps(run_prefill(ls, synth, wl, args.steps, args.warmup,
                                     n_rows_cpu=4 * args.cpu_sample)), flush=True)
        if args.copy_calib > 0:
            copy_calibration(args.copy_calib << 20)
        return
    if wl.serve_drift > 0:
        run_serve(ls, synth, wl, args)
        return
    headline = wl.name == "decode-128k-b32"
    result, probe_src = run_decode(ls, synth, wl, args.steps, args.warmup, args.replicas,
                                   full=True, n_single=2 if args.cpu_sample else 0,
                                   n_parallel=args.cpu_sample)
    result["copy_GBs"] = copy_bandwidth()
    result["read_probe"] = read_probes(ls, wl, *probe_src)
    del probe_src
    gc.collect()
    torch.cuda.empty_cache()
    if args.copy_calib > 0:
        copy_calibration(args.copy_calib << 20)
    if headline and args.extras:
        # the other workloads, each a sub-object with its own metric; their
        # inputs are built and freed in turn
        extra = {}
        # (the latency-bound single request is also timed as HIP-graph
        # replays: eager, the host's enqueue of its launches is on its path)
        for name, steps, warm, reps_, n1, npar, gr in (
                ("tiny-4k", 50, 20, 1, 1, 4, True),
                ("decode-16k-b192", 10, 4, 1, 1, 16, False),
                ("decode-950k-b4", 20, 20, 2, 0, 4, False)):
            sub, _ = run_decode(ls, synth, synth.WORKLOADS[name], steps, warm, reps_,
                                full=False, n_single=n1 if args.cpu_sample else 0,
                                n_parallel=npar if args.cpu_sample else 0, with_graph=gr)
            extra[name] = sub
            gc.collect()
            torch.cuda.empty_cache()
        extra["prefill-4k-128k"] = run_prefill(ls, synth, synth.WORKLOADS["prefill-4k-128k"], 3,
                                               1, n_rows_cpu=64 if args.cpu_sample else 0)
        gc.collect()
        torch.cuda.empty_cache()
        result["workloads"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
