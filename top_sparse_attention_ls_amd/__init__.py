"""Python binding of libls.so, the gfx950 sparse-decode library.

Argument marshalling only: every function here turns torch tensors into
device pointers and the current torch stream into a hipStream_t, and calls
the C-ABI declared in include/ls.h.  All computation happens in the HIP
kernels; there is no CPU fallback.  If the library is missing, load() raises.

Stages (see include/ls.h for the exact contracts):
  pack_coarse          compact 4-bit indexer keys (run when keys are appended)
  index_coarse         coarse scores of every token -> n_cand candidates
  refine_topk          exact int8 scores of the candidates -> top-k
  hot_gather           resolve against the hot buffer, copy misses from the pool
  sparse_attn_decode   attention over the selected rows
  DecodeStep           the whole step, one call (optionally with the original
                       keys on the host behind a key cache, and with both
                       caches committing)
  cache_commit         least-recently-used commit of one step's entries
  append_token         the new token's keys and KV row at ctx_len, ctx_len += 1
  prefill_index_topk / prefill_stream_layers   prefill-chunk indexer
  read_probe           memory-read bandwidth probe (measurement context only)
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libls.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "ls.h")

LS_OK, LS_E_ARG, LS_E_UNSUPPORTED, LS_E_WORKSPACE, LS_E_HIP = 0, -1, -2, -3, -4
OP_COARSE, OP_REFINE, OP_HOT, OP_ATTN, OP_STEP, OP_PREFILL = 1, 2, 3, 4, 5, 6
STEP_EVENTS = 7
ABI_VERSION = 5

_I32, _I64, _F32, _P = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class IdxDesc(ctypes.Structure):
    _fields_ = [(n, _I32) for n in ("batch", "max_ctx", "n_heads", "head_dim", "n_cand", "topk",
                                    "keys_on_host", "key_slots")]


class HotDesc(ctypes.Structure):
    _fields_ = [(n, _I32) for n in ("batch", "max_ctx", "topk", "hot_slots", "row_elems",
                                    "pool_on_host")]


class AttnDesc(ctypes.Structure):
    _fields_ = ([(n, _I32) for n in ("batch", "n_q_heads", "n_kv_heads", "qk_dim", "v_dim",
                                     "topk")]
                + [(n, _I64) for n in ("kv_rows_per_req", "kv_row_stride", "kv_head_stride")]
                + [("scale", _F32), ("n_splits", _I32)])


class CommitDesc(ctypes.Structure):
    _fields_ = [("hot", _I32), ("keys", _I32), ("now", ctypes.c_uint32)]


class StepDesc(ctypes.Structure):
    _fields_ = [("idx", IdxDesc), ("hot", HotDesc), ("attn", AttnDesc), ("use_hot", _I32),
                ("commit", CommitDesc)]


class AppendDesc(ctypes.Structure):
    _fields_ = [(n, _I32) for n in ("batch", "max_ctx", "head_dim", "row_elems", "keys_on_host",
                                    "pool_on_host")]


class StepIO(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "q_idx_dev", "w_idx_dev", "kc_dev", "k8_dev", "kpos2slot_dev", "kcache_dev",
        "ctx_len_dev", "cand_dev", "topk_dev",
        "topk_score_dev", "pos2slot_dev", "hot_kv_dev", "pool_kv_dev", "rows_dev", "n_miss_dev",
        "q_attn_dev", "k_cache_dev", "v_cache_dev", "out_dev", "lse_dev", "stage_events",
        "slot2pos_dev", "stamp_dev", "kslot2pos_dev", "kstamp_dev", "n_key_miss_dev",
        "now_dev")]


class PrefillDesc(ctypes.Structure):
    _fields_ = [(n, _I32) for n in ("n_query", "max_ctx", "q_pos0", "n_heads", "head_dim",
                                    "topk")]


_lib = None


def load():
    """Load libls.so (built in-tree by build()).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libls.so not built (%s); run python -m "
                           "top_sparse_attention_ls_amd.build" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    L.ls_abi_version.restype = _I32
    if L.ls_abi_version() != ABI_VERSION:
        raise RuntimeError("%s has ABI version %d, this binding expects %d; rebuild it"
                           % (LIB_PATH, L.ls_abi_version(), ABI_VERSION))
    L.ls_last_error.restype = ctypes.c_char_p
    L.ls_last_hip_error.restype = _I32
    L.ls_workspace_size.argtypes = [_I32, _P]
    L.ls_workspace_size.restype = ctypes.c_size_t
    L.ls_workspace_init.argtypes = [_P, ctypes.c_size_t, _P]
    L.ls_pack_coarse.argtypes = [_P, _P, _I64, _I32, _P]
    L.ls_index_coarse.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.ls_refine_topk.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                 _P]
    L.ls_hot_gather.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.ls_sparse_attn_decode.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.ls_decode_step.argtypes = [_P, _P, _P, ctypes.c_size_t, _P]
    L.ls_prefill_index_topk.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.ls_prefill_stream_layers.argtypes = [_P, _I32, _P, _P, _P, _P, _P, _P, _P,
                                           ctypes.c_size_t, _P, _P]
    L.ls_cache_commit.argtypes = [_I32, _I32, _I32, _I32, ctypes.c_uint32, _P, _P, _P, _P, _P,
                                  _P, _P]
    L.ls_append_token.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P]
    L.ls_read_probe.argtypes = [_P, ctypes.c_uint64, _P, _I64, _I32, _P, _P]
    L.ls_decode_step_noalloc.argtypes = [_P, _P, _P]
    for name in ("ls_cache_commit", "ls_append_token", "ls_pack_coarse", "ls_index_coarse",
                 "ls_refine_topk", "ls_hot_gather", "ls_sparse_attn_decode", "ls_decode_step",
                 "ls_prefill_index_topk", "ls_prefill_stream_layers", "ls_workspace_init",
                 "ls_read_probe", "ls_decode_step_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def header_symbols() -> list:
    """Names of every function declared in include/ls.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ls_[a-z0-9_]+)\s*\(", text)))


class LSError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("libls error %d: %s" % (code, msg))
        self.code = code


def _check(rc):
    if rc != LS_OK:
        raise LSError(rc, load().ls_last_error().decode())


def last_error() -> str:
    return load().ls_last_error().decode()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name, shape=None):
    """The library takes raw pointers and trusts the descriptor's sizes, so
    every tensor is checked against them here, before any launch."""
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))


def _need_rows(t, min_elems, name):
    if t.numel() < min_elems:
        raise ValueError("%s holds %d elements, the descriptor needs %d" % (name, t.numel(),
                                                                           min_elems))


# ---------------------------------------------------------------- workspace --

_ws_cache = {}


def workspace_size(op: int, desc) -> int:
    n = load().ls_workspace_size(op, ctypes.byref(desc))
    if n == 0:
        raise LSError(LS_E_ARG, last_error())
    return n


def workspace(op: int, desc, device) -> torch.Tensor:
    """A cleared workspace for (op, shapes), cached per device."""
    key = (op, bytes(desc), str(device))
    ws = _ws_cache.get(key)
    if ws is None:
        n = workspace_size(op, desc)
        ws = torch.empty(n, dtype=torch.uint8, device=device)
        _check(load().ls_workspace_init(_p(ws), n, _stream()))
        _ws_cache[key] = ws
    return ws


def new_workspace(op: int, desc, device) -> torch.Tensor:
    n = workspace_size(op, desc)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    _check(load().ls_workspace_init(_p(ws), n, _stream()))
    return ws


# ------------------------------------------------------------------- stages --

def pack_coarse(k8: torch.Tensor) -> torch.Tensor:
    """[..., D] int8 keys -> [..., D/2] uint8 compact keys."""
    _need(k8, torch.int8, "k8")
    d = k8.shape[-1]
    kc = torch.empty(k8.shape[:-1] + (d // 2,), dtype=torch.uint8, device=k8.device)
    _check(load().ls_pack_coarse(_p(k8), _p(kc), k8.numel() // d, d, _stream()))
    return kc


def idx_desc(q, keys_like_rows: int, n_cand: int, topk: int, keys_on_host: bool = False,
             key_slots: int = 0) -> IdxDesc:
    B, H, D = q.shape
    return IdxDesc(B, keys_like_rows, H, D, n_cand, topk, 1 if keys_on_host else 0, key_slots)


def index_coarse(q, w, kc, ctx_len, n_cand: int, topk: int = 1, ws=None) -> torch.Tensor:
    """q [B,H,D] int8, w [B,H] int8, kc [B,L,D/2] uint8, ctx_len [B] int32."""
    _need(q, torch.int8, "q")
    B, H, D = q.shape
    _need(w, torch.int8, "w", (B, H)), _need(kc, torch.uint8, "kc", (B, kc.shape[1], D // 2))
    _need(ctx_len, torch.int32, "ctx_len", (B,))
    d = idx_desc(q, kc.shape[1], n_cand, topk)
    ws = workspace(OP_COARSE, d, q.device) if ws is None else ws
    cand = torch.empty((q.shape[0], n_cand), dtype=torch.int32, device=q.device)
    _check(load().ls_index_coarse(ctypes.byref(d), _p(q), _p(w), _p(kc), _p(ctx_len), _p(cand),
                                  _p(ws), ws.numel(), _stream()))
    return cand


def _key_cache(kpos2slot, kcache, B, L, D):
    """Checks an optional key cache; returns its row count (0 without one)."""
    if (kpos2slot is None) != (kcache is None):
        raise ValueError("kpos2slot and kcache go together")
    if kcache is None:
        return 0
    _need(kpos2slot, torch.int32, "kpos2slot", (B, L))
    _need(kcache, torch.int8, "kcache", (B, kcache.shape[1], D))
    if not (kpos2slot.is_cuda and kcache.is_cuda):
        raise ValueError("the key cache and its slot table must be device memory")
    return kcache.shape[1]


def refine_topk(q, w, k8, cand, ctx_len, topk: int, ws=None, kpos2slot=None, kcache=None):
    """k8 [B,L,D] int8 on the device or in pinned host memory (read over PCIe,
    candidates' rows only); optional key cache kcache [B,S,D] int8 with its
    slot table kpos2slot [B,L] int32 (-1: not cached), both on the device.
    Returns (topk [B,topk] int32, scores [B,topk] int64)."""
    _need(q, torch.int8, "q")
    B, H, D = q.shape
    _need(w, torch.int8, "w", (B, H)), _need(k8, torch.int8, "k8", (B, k8.shape[1], D))
    _need(cand, torch.int32, "cand", (B, cand.shape[1]))
    _need(ctx_len, torch.int32, "ctx_len", (B,))
    S = _key_cache(kpos2slot, kcache, B, k8.shape[1], D)
    d = idx_desc(q, k8.shape[1], cand.shape[1], topk, keys_on_host=not k8.is_cuda, key_slots=S)
    ws = workspace(OP_REFINE, d, q.device) if ws is None else ws
    out = torch.empty((q.shape[0], topk), dtype=torch.int32, device=q.device)
    sc = torch.empty((q.shape[0], topk), dtype=torch.int64, device=q.device)
    _check(load().ls_refine_topk(ctypes.byref(d), _p(q), _p(w), _p(k8), _p(kpos2slot),
                                 _p(kcache), _p(cand), _p(ctx_len), _p(out), _p(sc), _p(ws),
                                 ws.numel(), _stream()))
    return out, sc


def hot_gather(topk, pos2slot, hot, pool, hot_slots: int, ws=None):
    """topk [B,K] int32, pos2slot [B,L] int32, hot [B,S+K,row] bf16 (updated in
    place), pool [B,L,row] bf16 (device or pinned host).  Returns (rows, n_miss)."""
    _need(topk, torch.int32, "topk")
    B, K = topk.shape
    _need(pool, torch.bfloat16, "pool")
    L, row = pool.shape[1], pool.shape[2]
    _need(pool, torch.bfloat16, "pool", (B, L, row))
    _need(pos2slot, torch.int32, "pos2slot", (B, L))
    _need(hot, torch.bfloat16, "hot", (B, hot_slots + K, row))
    d = HotDesc(B, pool.shape[1], K, hot_slots, hot.shape[2], 0 if pool.is_cuda else 1)
    ws = workspace(OP_HOT, d, topk.device) if ws is None else ws
    rows = torch.empty((B, K), dtype=torch.int32, device=topk.device)
    n_miss = torch.empty((B,), dtype=torch.int32, device=topk.device)
    _check(load().ls_hot_gather(ctypes.byref(d), _p(topk), _p(pos2slot), _p(hot), _p(pool),
                                _p(rows), _p(n_miss), _p(ws), ws.numel(), _stream()))
    return rows, n_miss


def attn_desc(q, topk: int, n_kv_heads: int, v_dim: int, kv_rows_per_req: int,
              kv_row_stride: int, kv_head_stride: int, scale: float, n_splits: int = 0):
    B, Hq, dqk = q.shape
    return AttnDesc(B, Hq, n_kv_heads, dqk, v_dim, topk, kv_rows_per_req, kv_row_stride,
                    kv_head_stride, float(scale), n_splits)


def sparse_attn_decode(q, k_base, v_base, rows, scale: float, n_kv_heads: int, v_dim: int,
                       kv_rows_per_req: int, kv_row_stride: int, kv_head_stride: int = 0,
                       n_splits: int = 0, ws=None):
    """q [B,Hq,qk_dim] bf16; rows [B,K] int32 (-1 ends a list).  K/V element
    (b, row r, kv head g, d) sits at base[(b*kv_rows_per_req + r)*kv_row_stride
    + g*kv_head_stride + d].  Returns (out [B,Hq,v_dim] bf16, lse [B,Hq] f32)."""
    _need(q, torch.bfloat16, "q"), _need(rows, torch.int32, "rows", (q.shape[0], rows.shape[1]))
    _need(k_base, torch.bfloat16, "k_base"), _need(v_base, torch.bfloat16, "v_base")
    last = (q.shape[0] * kv_rows_per_req - 1) * kv_row_stride + (n_kv_heads - 1) * kv_head_stride
    _need_rows(k_base, last + q.shape[2], "k_base")
    _need_rows(v_base, last + v_dim, "v_base")
    d = attn_desc(q, rows.shape[1], n_kv_heads, v_dim, kv_rows_per_req, kv_row_stride,
                  kv_head_stride, scale, n_splits)
    ws = workspace(OP_ATTN, d, q.device) if ws is None else ws
    B, Hq, _ = q.shape
    out = torch.empty((B, Hq, v_dim), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(load().ls_sparse_attn_decode(ctypes.byref(d), _p(q), _p(k_base), _p(v_base), _p(rows),
                                        _p(out), _p(lse), _p(ws), ws.numel(), _stream()))
    return out, lse


class DecodeStep:
    """One layer's decode step over a batch: fixed shapes, own workspace and
    output buffers.  run() enqueues the whole step on the current stream."""

    def __init__(self, *, batch, max_ctx, idx_heads, idx_dim, n_cand, topk, q_heads, qk_dim,
                 v_dim, scale, hot_slots=0, kv_heads=1, kv_row_stride=None, kv_head_stride=0,
                 pool_on_host=False, keys_on_host=False, key_slots=0, commit_hot=False,
                 commit_keys=False, n_splits=0, device="cuda"):
        self.use_hot = hot_slots > 0
        idx = IdxDesc(batch, max_ctx, idx_heads, idx_dim, n_cand, topk, 1 if keys_on_host else 0,
                      key_slots)
        row = qk_dim
        if self.use_hot:
            hot = HotDesc(batch, max_ctx, topk, hot_slots, row, 1 if pool_on_host else 0)
            attn = AttnDesc(batch, q_heads, 1, qk_dim, v_dim, topk, hot_slots + topk, row, 0,
                            float(scale), n_splits)
        else:
            hot = HotDesc(0, 0, 0, 0, 0, 0)
            stride = kv_row_stride if kv_row_stride is not None else kv_heads * qk_dim
            attn = AttnDesc(batch, q_heads, kv_heads, qk_dim, v_dim, topk, max_ctx, stride,
                            kv_head_stride, float(scale), n_splits)
        self.desc = StepDesc(idx, hot, attn, 1 if self.use_hot else 0,
                             CommitDesc(1 if commit_hot else 0, 1 if commit_keys else 0, 0))
        self.device = torch.device(device)
        self.ws = new_workspace(OP_STEP, self.desc, self.device)
        dev = self.device
        self.cand = torch.empty((batch, n_cand), dtype=torch.int32, device=dev)
        self.topk = torch.empty((batch, topk), dtype=torch.int32, device=dev)
        self.topk_score = torch.empty((batch, topk), dtype=torch.int64, device=dev)
        self.rows = torch.empty((batch, topk), dtype=torch.int32, device=dev)
        self.n_miss = torch.empty((batch,), dtype=torch.int32, device=dev)
        self.out = torch.empty((batch, q_heads, v_dim), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((batch, q_heads), dtype=torch.float32, device=dev)
        # candidates whose key came from k8 (written when the key cache commits)
        self.n_key_miss = torch.zeros((batch,), dtype=torch.int32, device=dev)

    def run(self, *, q_idx, w_idx, kc, k8, ctx_len, q_attn, pos2slot=None, hot_kv=None,
            pool_kv=None, k_cache=None, v_cache=None, kpos2slot=None, kcache=None,
            slot2pos=None, stamp=None, kslot2pos=None, kstamp=None, now=0, events=None,
            noalloc=False):
        """With commits, slot2pos / stamp (hot buffer) and kslot2pos / kstamp
        (key cache) are the caches' LRU state [B, slots] int32 (stamps held
        as uint32 bits), updated in place with pos2slot / kpos2slot; now is
        this step's stamp (see cache_commit), an int or a one-element int32
        device tensor read when the kernels run (for graph capture).
        noalloc: run ls_decode_step_noalloc, on the library's static scratch
        instead of this step's workspace."""
        i, a, h = self.desc.idx, self.desc.attn, self.desc.hot
        B, L, H, D = i.batch, i.max_ctx, i.n_heads, i.head_dim
        _need(q_idx, torch.int8, "q_idx", (B, H, D)), _need(w_idx, torch.int8, "w_idx", (B, H))
        _need(kc, torch.uint8, "kc", (B, L, D // 2)), _need(k8, torch.int8, "k8", (B, L, D))
        _need(ctx_len, torch.int32, "ctx_len", (B,))
        if k8.is_cuda == bool(i.keys_on_host):
            raise ValueError("k8 must be %s memory for this step" %
                             ("pinned host" if i.keys_on_host else "device"))
        if _key_cache(kpos2slot, kcache, B, L, D) != i.key_slots:
            raise ValueError("this step was built for a key cache of %d rows" % i.key_slots)
        _need(q_attn, torch.bfloat16, "q_attn", (B, a.n_q_heads, a.qk_dim))
        if self.use_hot:
            row = h.row_elems
            _need(pos2slot, torch.int32, "pos2slot", (B, L))
            _need(hot_kv, torch.bfloat16, "hot_kv", (B, h.hot_slots + i.topk, row))
            _need(pool_kv, torch.bfloat16, "pool_kv", (B, L, row))
            if pool_kv.is_cuda == bool(h.pool_on_host):
                raise ValueError("pool_kv must be %s memory for this step" %
                                 ("pinned host" if h.pool_on_host else "device"))
        else:
            _need(k_cache, torch.bfloat16, "k_cache"), _need(v_cache, torch.bfloat16, "v_cache")
            last = (B * a.kv_rows_per_req - 1) * a.kv_row_stride + \
                (a.n_kv_heads - 1) * a.kv_head_stride
            _need_rows(k_cache, last + a.qk_dim, "k_cache")
            _need_rows(v_cache, last + a.v_dim, "v_cache")
        io = StepIO()
        io.q_idx_dev, io.w_idx_dev = q_idx.data_ptr(), w_idx.data_ptr()
        io.kc_dev, io.k8_dev, io.ctx_len_dev = kc.data_ptr(), k8.data_ptr(), ctx_len.data_ptr()
        if i.key_slots:
            io.kpos2slot_dev, io.kcache_dev = kpos2slot.data_ptr(), kcache.data_ptr()
        io.cand_dev, io.topk_dev = self.cand.data_ptr(), self.topk.data_ptr()
        io.topk_score_dev = self.topk_score.data_ptr()
        if self.use_hot:
            io.pos2slot_dev, io.hot_kv_dev = pos2slot.data_ptr(), hot_kv.data_ptr()
            io.pool_kv_dev = pool_kv.data_ptr()
            io.rows_dev, io.n_miss_dev = self.rows.data_ptr(), self.n_miss.data_ptr()
        else:
            io.k_cache_dev, io.v_cache_dev = k_cache.data_ptr(), v_cache.data_ptr()
        io.q_attn_dev = q_attn.data_ptr()
        io.out_dev, io.lse_dev = self.out.data_ptr(), self.lse.data_ptr()
        c = self.desc.commit
        if isinstance(now, torch.Tensor):
            _need(now, torch.int32, "now", (1,))
            if not now.is_cuda:
                raise ValueError("a tensor now must be device memory")
            c.now, io.now_dev = 0, now.data_ptr()
        else:
            if (c.hot or c.keys) and not 0 < int(now) < 0xFFFFFFFF:
                raise ValueError("a committing step needs a stamp now in [1, 2^32 - 2] "
                                 "(0 marks a slot never used)")
            c.now = int(now) & 0xFFFFFFFF
        if c.hot:
            S = h.hot_slots
            _need(slot2pos, torch.int32, "slot2pos", (B, S)), _need(stamp, torch.int32, "stamp",
                                                                    (B, S))
            io.slot2pos_dev, io.stamp_dev = slot2pos.data_ptr(), stamp.data_ptr()
        if c.keys:
            S = i.key_slots
            _need(kslot2pos, torch.int32, "kslot2pos", (B, S))
            _need(kstamp, torch.int32, "kstamp", (B, S))
            io.kslot2pos_dev, io.kstamp_dev = kslot2pos.data_ptr(), kstamp.data_ptr()
            io.n_key_miss_dev = self.n_key_miss.data_ptr()
        if events is not None:  # STEP_EVENTS torch events; None entries are skipped
            arr = (ctypes.c_void_p * STEP_EVENTS)(*[e.cuda_event if e is not None else None
                                                    for e in events])
            io.stage_events = ctypes.cast(arr, ctypes.c_void_p)
        if noalloc:
            _check(load().ls_decode_step_noalloc(ctypes.byref(self.desc), ctypes.byref(io),
                                                 _stream()))
        else:
            _check(load().ls_decode_step(ctypes.byref(self.desc), ctypes.byref(io),
                                         _p(self.ws), self.ws.numel(), _stream()))
        return self.out, self.lse


# ------------------------------------------------------------- cache state --

def cache_commit(entries, pos2slot, slot2pos, stamp, now: int):
    """Least-recently-used commit of the entries [B, n] (ascending positions,
    -1 padded) into per-request caches of S slots: pos2slot [B, L] int32,
    slot2pos [B, S] int32, stamp [B, S] int32 holding uint32 stamps, updated
    in place.  Returns (dst [B, n] int32, n_inserted [B] int32)."""
    _need(entries, torch.int32, "entries")
    B, n = entries.shape
    _need(pos2slot, torch.int32, "pos2slot", (B, pos2slot.shape[1]))
    S = slot2pos.shape[1]
    _need(slot2pos, torch.int32, "slot2pos", (B, S)), _need(stamp, torch.int32, "stamp", (B, S))
    dst = torch.empty((B, n), dtype=torch.int32, device=entries.device)
    n_ins = torch.empty((B,), dtype=torch.int32, device=entries.device)
    _check(load().ls_cache_commit(B, pos2slot.shape[1], S, n, int(now) & 0xFFFFFFFF, _p(entries),
                                  _p(pos2slot), _p(slot2pos), _p(stamp), _p(dst), _p(n_ins),
                                  _stream()))
    return dst, n_ins


def append_token(new_k8, k8, kc, ctx_len, new_kv=None, pool=None):
    """Writes each request's new token at position ctx_len[b] (if below
    max_ctx) and advances ctx_len: new_k8 [B, D] int8 into k8 [B, L, D] and
    its compact form into kc [B, L, D/2]; new_kv [B, row] bf16 into pool
    [B, L, row].  k8 and pool may be pinned host memory."""
    _need(new_k8, torch.int8, "new_k8")
    B, D = new_k8.shape
    _need(k8, torch.int8, "k8", (B, k8.shape[1], D))
    L = k8.shape[1]
    _need(kc, torch.uint8, "kc", (B, L, D // 2)), _need(ctx_len, torch.int32, "ctx_len", (B,))
    row = 0
    if (new_kv is None) != (pool is None):
        raise ValueError("new_kv and pool go together")
    if pool is not None:
        row = pool.shape[2]
        _need(new_kv, torch.bfloat16, "new_kv", (B, row))
        _need(pool, torch.bfloat16, "pool", (B, L, row))
    d = AppendDesc(B, L, D, row, 0 if k8.is_cuda else 1,
                   0 if (pool is None or pool.is_cuda) else 1)
    _check(load().ls_append_token(ctypes.byref(d), _p(new_k8), _p(new_kv), _p(k8), _p(kc),
                                  _p(pool), _p(ctx_len), _stream()))


# ------------------------------------------------------------------ prefill --

def prefill_desc(q, max_ctx: int, q_pos0: int, topk: int) -> PrefillDesc:
    Tq, H, D = q.shape
    return PrefillDesc(Tq, max_ctx, q_pos0, H, D, topk)


def prefill_index_topk(q, w, keys, q_pos0: int, topk: int, ws=None) -> torch.Tensor:
    """q [Tq,H,D] int8, w [Tq,H] int8, keys [L,D] int8 on the device.  Query i
    sits at absolute position q_pos0 + i and sees keys 0..q_pos0+i.  Returns
    topk [Tq, topk] int32, ascending, -1 padded."""
    _need(q, torch.int8, "q")
    Tq, H, D = q.shape
    _need(w, torch.int8, "w", (Tq, H)), _need(keys, torch.int8, "keys", (keys.shape[0], D))
    d = prefill_desc(q, keys.shape[0], q_pos0, topk)
    ws = workspace(OP_PREFILL, d, q.device) if ws is None else ws
    out = torch.empty((Tq, topk), dtype=torch.int32, device=q.device)
    _check(load().ls_prefill_index_topk(ctypes.byref(d), _p(q), _p(w), _p(keys), _p(out),
                                        _p(ws), ws.numel(), _stream()))
    return out


def prefill_stream_layers(qs, ws_, keys_host, q_pos0: int, topk: int, buf0=None, buf1=None,
                          copy_stream=None, ws=None):
    """Layers l = 0..n-1: qs[l] [Tq,H,D] int8 and ws_[l] [Tq,H] int8 on the
    device, keys_host[l] [L,D] int8 in pinned host memory.  The histories are
    copied through the two device buffers buf0 / buf1 on copy_stream while
    the indexer runs on the current stream.  Returns the per-layer top-k."""
    n = len(qs)
    Tq, H, D = qs[0].shape
    L = keys_host[0].shape[0]
    for l in range(n):
        _need(qs[l], torch.int8, "q[%d]" % l, (Tq, H, D))
        _need(ws_[l], torch.int8, "w[%d]" % l, (Tq, H))
        _need(keys_host[l], torch.int8, "keys[%d]" % l, (L, D))
        if keys_host[l].is_cuda or not keys_host[l].is_pinned():
            raise ValueError("keys[%d] must be pinned host memory" % l)
    dev = qs[0].device
    buf0 = torch.empty((L, D), dtype=torch.int8, device=dev) if buf0 is None else buf0
    buf1 = torch.empty((L, D), dtype=torch.int8, device=dev) if buf1 is None else buf1
    _need(buf0, torch.int8, "buf0", (L, D)), _need(buf1, torch.int8, "buf1", (L, D))
    copy_stream = torch.cuda.Stream(device=dev) if copy_stream is None else copy_stream
    # the buffers are written on the copy stream: keep the allocator from
    # handing their memory out again before that stream is done with them
    buf0.record_stream(copy_stream)
    buf1.record_stream(copy_stream)
    d = prefill_desc(qs[0], L, q_pos0, topk)
    ws = workspace(OP_PREFILL, d, dev) if ws is None else ws
    outs = [torch.empty((Tq, topk), dtype=torch.int32, device=dev) for _ in range(n)]

    def arr(ts):
        return (ctypes.c_void_p * n)(*[t.data_ptr() for t in ts])

    _check(load().ls_prefill_stream_layers(ctypes.byref(d), n, arr(qs), arr(ws_), arr(keys_host),
                                           _p(buf0), _p(buf1), arr(outs), _p(ws), ws.numel(),
                                           _stream(), ctypes.c_void_p(copy_stream.cuda_stream)))
    return outs


def read_probe(base, rows=None, row_bytes=0, sink=None):
    """ls_read_probe: a streaming read of the whole tensor base (rows None) or
    a gather of the rows rows (int32, device) of row_bytes each; returns the
    sink word (a device tensor, for the caller to synchronise on)."""
    if not base.is_cuda or not base.is_contiguous():
        raise ValueError("base must be a contiguous device tensor")
    if sink is None:
        sink = torch.zeros((1,), dtype=torch.int32, device=base.device)
    nbytes = base.numel() * base.element_size()
    if rows is not None:
        _need(rows, torch.int32, "rows")
        n, rp = rows.numel(), _p(rows)
    else:
        n, rp = 0, None
    _check(load().ls_read_probe(_p(base), nbytes, rp, n, int(row_bytes), _p(sink), _stream()))
    return sink
