"""Seeded synthetic inputs for the decode step and the prefill indexer.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle's tests.  It holds none of the method's arithmetic: no scoring, no
compact-key packing, no selection, no attention.  It only draws tensors and
lays out the caller-owned cache state (hot buffer, slot table) from a
selection that the caller passes in.

Distributions (the library's workload recipe):
  * indexer query and keys: round-half-even(N(0, 24)) clipped to [-127, 127],
    int8; per-head weights uniform integers in [1, 16];
  * planted tokens: key[d] = 100 * sign(sum_h w[h] * q[h][d]) -- the sign
    pattern of the head-weighted query, so that every head's ReLU term rises
    together;
  * attention query and cached rows: N(0, 1) rounded to bfloat16 (RNE);
  * hot buffer: a given fraction of the selected tokens is made resident at
    random slots, the remaining slots hold random unselected tokens, and the
    rest of the selection must be fetched from the pool.

Every tensor is drawn from its own generator seeded by (workload seed,
tensor id, sub-index), so no tensor depends on the order of generation.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

# tensor ids for seeding
(T_QIDX, T_WIDX, T_KEYS, T_PLANT, T_QATT, T_POOL, T_HOT, T_KCACHE, T_VCACHE, T_RAGGED,
 T_KEYCACHE) = range(11)


@dataclass(frozen=True)
class Workload:
    """Shapes of one workload.  attn = "mla" (one shared latent row per token,
    V = its first v_dim elements) or "mha" (separate K and V per kv head)."""
    name: str
    seed: int
    batch: int
    ctx: int
    idx_heads: int
    idx_dim: int
    n_cand: int
    topk: int
    planted: int = 0                 # number of planted tokens per request (or per layer)
    bursts: tuple = ()               # (n_bursts, burst_len): planted tokens in bursts
    attn: str = "mla"
    q_heads: int = 128
    kv_heads: int = 1
    qk_dim: int = 576
    v_dim: int = 512
    scale: float = 1.0 / math.sqrt(192.0)
    hot_slots: int = 0               # 0: no hot buffer
    miss_rate: float = 0.0
    pool_on_host: bool = False
    keys_on_host: bool = False       # original int8 keys in pinned host memory
    key_slots: int = 0               # rows of the per-request indexer-key cache (0: none)
    key_miss_rate: float = 0.0       # share of the candidates whose key is not cached
    # multi-step serving: both caches commit each step, a token is appended,
    # and the indexer query drifts (each element redrawn with this rate)
    serve_drift: float = 0.0
    serve_microbatches: int = 1      # micro-batches on their own streams in the serving loop
    # prefill only
    n_query: int = 0
    layers: int = 0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # single-layer decode step, one request of 4096 tokens, MHA, no hot buffer
    "tiny-4k": Workload("tiny-4k", 1000, batch=1, ctx=4096, idx_heads=4, idx_dim=64,
                        n_cand=1024, topk=256, planted=16, attn="mha", q_heads=8,
                        kv_heads=8, qk_dim=64, v_dim=64, scale=1.0 / 8.0),
    # decode at 128K context, 32 requests, MLA latent 576, 20% hot-buffer miss (HBM pool)
    "decode-128k-b32": Workload("decode-128k-b32", 1001, batch=32, ctx=131072,
                                idx_heads=64, idx_dim=128, n_cand=8192, topk=2048,
                                planted=1310, hot_slots=4096, miss_rate=0.2),
    # decode at 16K context, 192 requests, 40% miss from a pinned host pool
    "decode-16k-b192": Workload("decode-16k-b192", 1002, batch=192, ctx=16384,
                                idx_heads=64, idx_dim=128, n_cand=4096, topk=2048,
                                planted=163, hot_slots=4096, miss_rate=0.4,
                                pool_on_host=True),
    # the same step with the original int8 keys off the GPU (pinned host) and
    # a 16384-row indexer-key cache per request that holds 80% of the step's
    # candidates
    "decode-128k-b32-hostkeys": Workload("decode-128k-b32-hostkeys", 1001, batch=32,
                                         ctx=131072, idx_heads=64, idx_dim=128, n_cand=8192,
                                         topk=2048, planted=1310, hot_slots=4096,
                                         miss_rate=0.2, keys_on_host=True, key_slots=16384,
                                         key_miss_rate=0.2),
    # serving: steps in a row over the host-keys layout, both caches starting
    # empty and committing every step, one token appended per step and
    # request, the indexer query drifting by 10% of its elements per step
    "decode-128k-b32-serve": Workload("decode-128k-b32-serve", 1001, batch=32, ctx=131072,
                                      idx_heads=64, idx_dim=128, n_cand=8192, topk=2048,
                                      planted=1310, hot_slots=4096, keys_on_host=True,
                                      key_slots=16384, serve_drift=0.1),
    # the serving loop over a stack of four layers (each its own state)
    "decode-128k-b32-serve-4l": Workload("decode-128k-b32-serve-4l", 1001, batch=32,
                                         ctx=131072, idx_heads=64, idx_dim=128, n_cand=8192,
                                         topk=2048, planted=1310, hot_slots=4096,
                                         keys_on_host=True, key_slots=16384, serve_drift=0.1,
                                         layers=4),
    # decode near 1M context, 4 requests, planted tokens in 8 bursts of 512
    "decode-950k-b4": Workload("decode-950k-b4", 1003, batch=4, ctx=950000, idx_heads=64,
                               idx_dim=128, n_cand=16384, topk=2048, bursts=(8, 512),
                               hot_slots=4096, miss_rate=0.2),
    # prefill chunk: 4096 query tokens (the last 4096 positions) over 131072 keys, 4 layers
    "prefill-4k-128k": Workload("prefill-4k-128k", 1004, batch=1, ctx=131072, idx_heads=64,
                                idx_dim=128, n_cand=0, topk=2048, planted=1310,
                                n_query=4096, layers=4),
}


def generator(seed: int, tensor_id: int, sub: int, device) -> torch.Generator:
    """Independent generator for (workload seed, tensor id, sub-index)."""
    state = np.random.SeedSequence([int(seed), int(tensor_id), int(sub)]).generate_state(
        2, dtype=np.uint32)
    g = torch.Generator(device=device)
    g.manual_seed(int(state[0]) | (int(state[1]) << 32) & ((1 << 63) - 1))
    return g


def int8_normal(shape, std: float, g: torch.Generator, device) -> torch.Tensor:
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
    return torch.round(z).clamp_(-127, 127).to(torch.int8)


def bf16_normal(shape, g: torch.Generator, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def planted_pattern(q: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """[H, D] int8 query and [H] weights -> [D] int8 key 100*sign(sum_h w_h q_h)."""
    s = (w.to(torch.int32)[:, None] * q.to(torch.int32)).sum(0)
    return (torch.sign(s) * 100).to(torch.int8)


def planted_positions(wl: Workload, ctx: int, g: torch.Generator, device) -> torch.Tensor:
    if wl.bursts:
        n_b, blen = wl.bursts
        # sorted uniform starts in [0, ctx - n_b*blen], then shifted so bursts never overlap
        starts = torch.sort(torch.randint(0, ctx - n_b * blen + 1, (n_b,), generator=g,
                                          device=device)).values
        starts = starts + torch.arange(n_b, device=device) * blen
        return (starts[:, None] + torch.arange(blen, device=device)[None, :]).reshape(-1)
    n = min(wl.planted, ctx)
    return torch.randperm(ctx, generator=g, device=device)[:n]


def indexer_inputs(wl: Workload, device, ctx_len=None, batch=None, ctx=None):
    """q [B,H,D] int8, w [B,H] int8, keys [B,max_ctx,D] int8, planted list."""
    B = wl.batch if batch is None else batch
    L = wl.ctx if ctx is None else ctx
    H, D = wl.idx_heads, wl.idx_dim
    q = torch.empty((B, H, D), dtype=torch.int8, device=device)
    w = torch.empty((B, H), dtype=torch.int8, device=device)
    keys = torch.empty((B, L, D), dtype=torch.int8, device=device)
    planted = []
    for b in range(B):
        q[b] = int8_normal((H, D), 24.0, generator(wl.seed, T_QIDX, b, device), device)
        w[b] = torch.randint(1, 17, (H,), generator=generator(wl.seed, T_WIDX, b, device),
                             device=device, dtype=torch.int32).to(torch.int8)
        keys[b] = int8_normal((L, D), 24.0, generator(wl.seed, T_KEYS, b, device), device)
        n_valid = L if ctx_len is None else int(ctx_len[b])
        pp = planted_positions(wl, max(n_valid, 1), generator(wl.seed, T_PLANT, b, device),
                               device) if n_valid > 0 else torch.empty(0, dtype=torch.int64,
                                                                       device=device)
        if pp.numel():
            keys[b, pp] = planted_pattern(q[b], w[b])
        planted.append(pp)
    return dict(q=q, w=w, keys=keys, planted=planted)


def prefill_inputs(wl: Workload, layer: int, device, n_query=None, ctx=None):
    """One layer of the prefill chunk: q [Tq,H,D], w [Tq,H], keys [L,D] (int8)."""
    Tq = wl.n_query if n_query is None else n_query
    L = wl.ctx if ctx is None else ctx
    H, D = wl.idx_heads, wl.idx_dim
    sub = 1000 * layer
    q = int8_normal((Tq, H, D), 24.0, generator(wl.seed, T_QIDX, sub, device), device)
    w = torch.randint(1, 17, (Tq, H), generator=generator(wl.seed, T_WIDX, sub, device),
                      device=device, dtype=torch.int32).to(torch.int8)
    keys = int8_normal((L, D), 24.0, generator(wl.seed, T_KEYS, sub, device), device)
    g = generator(wl.seed, T_PLANT, sub, device)
    n_p = min(max(wl.planted * L // max(wl.ctx, 1), 1), L)
    pos = torch.randperm(L, generator=g, device=device)[:n_p]
    src = torch.randint(0, Tq, (n_p,), generator=g, device=device)
    # each planted key copies the sign pattern of a query row of the chunk
    s = (w.to(torch.int32)[src][:, :, None] * q.to(torch.int32)[src]).sum(1)
    keys[pos] = (torch.sign(s) * 100).to(torch.int8)
    return dict(q=q, w=w, keys=keys)


def attention_query(wl: Workload, device, batch=None):
    B = wl.batch if batch is None else batch
    out = torch.empty((B, wl.q_heads, wl.qk_dim), dtype=torch.bfloat16, device=device)
    for b in range(B):
        out[b] = bf16_normal((wl.q_heads, wl.qk_dim), generator(wl.seed, T_QATT, b, device),
                             device)
    return out


def kv_pool(wl: Workload, device, batch=None, ctx=None, pin=False, gen_device=None):
    """MLA full-history pool [B, L, qk_dim] bf16 (one latent row per token).
    With pin=True the pool is allocated in pinned host memory (drawn on
    gen_device, default the host, and copied row block by row block)."""
    B = wl.batch if batch is None else batch
    L = wl.ctx if ctx is None else ctx
    gdev = device if gen_device is None else gen_device
    if pin:
        out = torch.empty((B, L, wl.qk_dim), dtype=torch.bfloat16, pin_memory=True)
    else:
        out = torch.empty((B, L, wl.qk_dim), dtype=torch.bfloat16, device=device)
    for b in range(B):
        out[b].copy_(bf16_normal((L, wl.qk_dim), generator(wl.seed, T_POOL, b, gdev), gdev))
    return out


def kv_cache_mha(wl: Workload, device, batch=None, ctx=None):
    """MHA caches K, V: [B, L, kv_heads, head_dim] bf16."""
    B = wl.batch if batch is None else batch
    L = wl.ctx if ctx is None else ctx
    shp = (L, wl.kv_heads, wl.qk_dim)
    k = torch.empty((B,) + shp, dtype=torch.bfloat16, device=device)
    v = torch.empty((B, L, wl.kv_heads, wl.v_dim), dtype=torch.bfloat16, device=device)
    for b in range(B):
        k[b] = bf16_normal(shp, generator(wl.seed, T_KCACHE, b, device), device)
        v[b] = bf16_normal((L, wl.kv_heads, wl.v_dim), generator(wl.seed, T_VCACHE, b, device),
                           device)
    return k, v


def hot_fill(wl: Workload, selected: torch.Tensor, pool: torch.Tensor, device,
             miss_rate=None, hot_slots=None, ctx=None, scratch=None):
    """Lay out the hot buffer so that a fixed share of a known selection misses.

    selected: [B, n] int32 selected positions per request (-1 padding), as
    computed by the caller.  scratch: rows reserved for the step's misses
    after the slots (the step's top-k; default n).  For each request, round(rate * n_sel) selected
    tokens are left out; the others are made resident at random distinct
    slots, and the remaining slots hold random unselected tokens.  Resident
    rows are byte copies of the pool rows; the k scratch rows after the slots
    start zeroed.
    Returns pos2slot [B, L] int32, hot [B, S + scratch, row] bf16, n_miss list."""
    rate = wl.miss_rate if miss_rate is None else miss_rate
    S = wl.hot_slots if hot_slots is None else hot_slots
    B, n = selected.shape
    k = n if scratch is None else scratch
    L = pool.shape[1] if ctx is None else ctx
    row = pool.shape[2]
    sel_cpu = selected.to("cpu")
    pos2slot = torch.full((B, L), -1, dtype=torch.int32, device=device)
    hot = torch.zeros((B, S + k, row), dtype=torch.bfloat16, device=device)
    n_miss = []
    for b in range(B):
        g = generator(wl.seed, T_HOT, b, "cpu")
        valid = sel_cpu[b][sel_cpu[b] >= 0].to(torch.int64)
        n_sel = int(valid.numel())
        nm = int(math.floor(rate * n_sel + 0.5))
        n_hit = n_sel - nm
        hits = valid[torch.randperm(n_sel, generator=g)[:n_hit]]
        slots = torch.randperm(S, generator=g)
        mask = torch.ones(L, dtype=torch.bool)
        mask[valid] = False
        others = torch.randperm(L, generator=g)
        others = others[mask[others]][: max(S - n_hit, 0)]
        res_pos = torch.cat([hits, others])
        res_slot = slots[: res_pos.numel()].to(torch.int32)
        pos2slot[b, res_pos.to(device)] = res_slot.to(device)
        src = pool[b].index_select(0, res_pos.to(pool.device))
        hot[b, res_slot.to(torch.int64).to(device)] = src.to(device)
        n_miss.append(nm)
    return pos2slot, hot, n_miss


def key_cache_fill(wl: Workload, cand: torch.Tensor, keys: torch.Tensor, device,
                   miss_rate=None, key_slots=None):
    """Lay out the indexer-key cache so that a fixed share of a known
    candidate set misses it.

    cand: [B, n] int32 candidate positions per request (-1 padding), as
    computed by the caller; keys: [B, L, D] int8 (any device).  For each
    request, round(rate * n_valid) candidates are left out; the others are
    made resident at random distinct rows, and the remaining rows hold
    random non-candidate tokens.  Cached rows are byte copies of the keys.
    Returns kpos2slot [B, L] int32, kcache [B, S, D] int8, n_key_miss list."""
    rate = wl.key_miss_rate if miss_rate is None else miss_rate
    S = wl.key_slots if key_slots is None else key_slots
    B, n = cand.shape
    L, D = keys.shape[1], keys.shape[2]
    cand_cpu = cand.to("cpu")
    kpos2slot = torch.full((B, L), -1, dtype=torch.int32, device=device)
    kcache = torch.zeros((B, S, D), dtype=torch.int8, device=device)
    n_miss = []
    for b in range(B):
        g = generator(wl.seed, T_KEYCACHE, b, "cpu")
        valid = cand_cpu[b][cand_cpu[b] >= 0].to(torch.int64)
        n_val = int(valid.numel())
        nm = int(math.floor(rate * n_val + 0.5))
        n_hit = n_val - nm
        if n_hit > S:
            raise ValueError("a key cache of %d rows cannot hold %d candidates" % (S, n_hit))
        hits = valid[torch.randperm(n_val, generator=g)[:n_hit]]
        rows = torch.randperm(S, generator=g)
        mask = torch.ones(L, dtype=torch.bool)
        mask[valid] = False
        others = torch.randperm(L, generator=g)
        others = others[mask[others]][: max(S - n_hit, 0)]
        res_pos = torch.cat([hits, others])
        res_row = rows[: res_pos.numel()].to(torch.int32)
        kpos2slot[b, res_pos.to(device)] = res_row.to(device)
        src = keys[b].index_select(0, res_pos.to(keys.device))
        kcache[b, res_row.to(torch.int64).to(device)] = src.to(device)
        n_miss.append(nm)
    return kpos2slot, kcache, n_miss


def drift_query(q: torch.Tensor, rate: float, g: torch.Generator, device) -> torch.Tensor:
    """The next decode step's indexer query: each element redrawn from the
    query distribution with probability rate (a synthetic model of how a
    request's selection carries over from step to step)."""
    fresh = int8_normal(q.shape, 24.0, g, device)
    keep = torch.rand(q.shape, generator=g, device=device) >= rate
    return torch.where(keep, q, fresh)


def ragged_lengths(wl: Workload, batch: int, max_ctx: int, min_ctx: int = 0) -> list:
    g = generator(wl.seed, T_RAGGED, 0, "cpu")
    return torch.randint(min_ctx, max_ctx + 1, (batch,), generator=g).tolist()
