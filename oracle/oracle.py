"""Python face of the plain CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports, links
or runs anything here, and nothing here imports the HIP library.

Every function marshals numpy arrays into the C oracle; the arithmetic lives
in ``oracle.c`` (single-threaded plain loops, int64 for indexer work, double
for attention).  Sources are cited there; the method comes from the LeanSparse
abstract (coarse-to-fine indexing, prefill layer streaming), the XM-Sparse
digest (hot KV buffer, fetch only the selected misses) and the dynamic sparse
attention abstract (attention over a top-k subset of cached rows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc -O2 (plain C, no OpenMP, no intrinsics)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_D = ctypes.c_double


def _declare(L):
    L.orc_coarse_value.argtypes = [_I32]
    L.orc_coarse_value.restype = _I32
    L.orc_pack_coarse.argtypes = [_P, _P, _I64, _I32]
    L.orc_unpack_coarse.argtypes = [_P, _P, _I64, _I32]
    L.orc_index_scores.argtypes = [_P, _P, _I32, _I32, _P, _I64, _I32, _P]
    L.orc_index_scores_at.argtypes = [_P, _P, _I32, _I32, _P, _P, _I64, _I32, _P]
    L.orc_select_top.argtypes = [_P, _P, _I64, _I64, _P, _P]
    L.orc_select_top.restype = _I64
    L.orc_hot_resolve.argtypes = [_P, _I32, _P, _I32, _P, _P]
    L.orc_hot_resolve.restype = _I32
    L.orc_hot_gather.argtypes = [_P, _I64, _P, _I32, _P, _I32]
    L.orc_cache_commit.argtypes = [_P, _I32, _I32, ctypes.c_uint32, _P, _I64, _P, _P, _P]
    L.orc_cache_commit.restype = _I32
    L.orc_attention.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P, _I64, _I64, _P, _I32,
                                _D, _P, _P]
    L.orc_decode_request.argtypes = [_P, _P, _I32, _I32, _P, _I32, _I32, _I32, _P, _I32,
                                     _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _I64, _I64,
                                     _D, _P, _P, _P, _P, _P, _P]
    L.orc_decode_request.restype = _I32
    L.orc_prefill_row.argtypes = [_P, _P, _I32, _I32, _P, _I32, _I32, _P, _P]
    L.orc_prefill_row.restype = _I64


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ keys --

def coarse_value(k: int) -> int:
    """floor(k / 16): the compact value of one int8 key element."""
    return int(lib().orc_coarse_value(int(k)))


def pack_coarse(k: np.ndarray) -> np.ndarray:
    """[..., D] int8 keys -> [..., D/2] bytes of signed nibbles (even d low)."""
    k = _c(k, np.int8)
    d = k.shape[-1]
    rows = int(np.prod(k.shape[:-1])) if k.ndim > 1 else 1
    out = np.empty(k.shape[:-1] + (d // 2,), dtype=np.uint8)
    lib().orc_pack_coarse(_ptr(k), _ptr(out), rows, d)
    return out


def unpack_coarse(kc: np.ndarray) -> np.ndarray:
    kc = _c(kc, np.uint8)
    half = kc.shape[-1]
    rows = int(np.prod(kc.shape[:-1])) if kc.ndim > 1 else 1
    out = np.empty(kc.shape[:-1] + (2 * half,), dtype=np.int8)
    lib().orc_unpack_coarse(_ptr(kc), _ptr(out), rows, 2 * half)
    return out


# --------------------------------------------------------------- scoring --

def index_scores(q: np.ndarray, w: np.ndarray, keys: np.ndarray, coarse: bool,
                 n_keys: int | None = None) -> np.ndarray:
    """Scores of keys[0:n_keys] for one request. q [H,D], w [H], keys [L,D]."""
    q, w, keys = _c(q, np.int8), _c(w, np.int8), _c(keys, np.int8)
    h, d = q.shape
    n = keys.shape[0] if n_keys is None else int(n_keys)
    out = np.empty(n, dtype=np.int64)
    lib().orc_index_scores(_ptr(q), _ptr(w), h, d, _ptr(keys), n, int(coarse), _ptr(out))
    return out


def index_scores_at(q, w, keys, pos, coarse: bool) -> np.ndarray:
    q, w, keys, pos = _c(q, np.int8), _c(w, np.int8), _c(keys, np.int8), _c(pos, np.int32)
    h, d = q.shape
    out = np.empty(pos.shape[0], dtype=np.int64)
    lib().orc_index_scores_at(_ptr(q), _ptr(w), h, d, _ptr(keys), _ptr(pos), pos.shape[0],
                              int(coarse), _ptr(out))
    return out


def select_top(score: np.ndarray, pos: np.ndarray, m: int):
    """Keep the m best by (score desc, pos asc); returns (pos asc, their scores)."""
    score, pos = _c(score, np.int64), _c(pos, np.int32)
    n = score.shape[0]
    kept = max(0, min(int(m), n))
    out_p = np.empty(max(kept, 1), dtype=np.int32)
    out_s = np.empty(max(kept, 1), dtype=np.int64)
    got = lib().orc_select_top(_ptr(score), _ptr(pos), n, int(m), _ptr(out_p), _ptr(out_s))
    assert got == kept
    return out_p[:kept], out_s[:kept]


def pad(a: np.ndarray, n: int, value) -> np.ndarray:
    out = np.full(n, value, dtype=a.dtype)
    out[: a.shape[0]] = a
    return out


# ------------------------------------------------------------ hot buffer --

def hot_resolve(sel: np.ndarray, pos2slot: np.ndarray, hot_slots: int):
    """Returns (rows [n_sel], miss_pos [n_miss])."""
    sel, p2s = _c(sel, np.int32), _c(pos2slot, np.int32)
    rows = np.empty(max(sel.shape[0], 1), dtype=np.int32)
    miss = np.empty(max(sel.shape[0], 1), dtype=np.int32)
    n_miss = lib().orc_hot_resolve(_ptr(sel), sel.shape[0], _ptr(p2s), int(hot_slots),
                                   _ptr(rows), _ptr(miss))
    return rows[: sel.shape[0]], miss[:n_miss]


def hot_gather(pool: np.ndarray, miss_pos: np.ndarray, hot: np.ndarray, hot_slots: int):
    """In place: hot[hot_slots + j] = pool[miss_pos[j]] (byte copies of rows)."""
    assert pool.flags.c_contiguous and hot.flags.c_contiguous
    row_bytes = pool.strides[0]
    assert hot.strides[0] == row_bytes
    mp = _c(miss_pos, np.int32)
    lib().orc_hot_gather(_ptr(pool), row_bytes, _ptr(mp), mp.shape[0], _ptr(hot), int(hot_slots))


def cache_commit(pos: np.ndarray, n_slots: int, now: int, pos2slot: np.ndarray,
                 slot2pos: np.ndarray, stamp: np.ndarray):
    """Least-recently-used commit of one step's entries into one request's
    cache (see orc_cache_commit).  pos2slot [L] int32, slot2pos [n_slots]
    int32 and stamp [n_slots] uint32 are updated in place (they must be
    contiguous arrays of those types).  Returns (dst [n] int32, n_inserted)."""
    for a, t in ((pos2slot, np.int32), (slot2pos, np.int32), (stamp, np.uint32)):
        assert a.dtype == t and a.flags.c_contiguous
    assert slot2pos.shape[0] == stamp.shape[0] == n_slots
    p = _c(pos, np.int32)
    dst = np.empty(max(p.shape[0], 1), np.int32)
    n_ins = lib().orc_cache_commit(_ptr(p), p.shape[0], int(n_slots), int(now), _ptr(pos2slot),
                                   pos2slot.shape[0], _ptr(slot2pos), _ptr(stamp), _ptr(dst))
    return dst[: p.shape[0]], int(n_ins)


# ------------------------------------------------------------- attention --

def attention(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, rows: np.ndarray,
              scale: float, n_kv_heads: int, v_dim: int, row_stride: int,
              head_stride: int):
    """One request. q_bits [Hq, qk_dim] uint16 (bf16 bits); k_bits / v_bits are
    flat uint16 arrays addressed as base[row*row_stride + g*head_stride + d].
    Returns (out [Hq, v_dim] float64, lse [Hq] float64)."""
    q = _c(q_bits, np.uint16)
    kb, vb = _c(k_bits, np.uint16), _c(v_bits, np.uint16)
    r = _c(rows, np.int32)
    hq, dqk = q.shape
    out = np.empty((hq, v_dim), dtype=np.float64)
    lse = np.empty(hq, dtype=np.float64)
    lib().orc_attention(_ptr(q), hq, int(n_kv_heads), dqk, int(v_dim), _ptr(kb), _ptr(vb),
                        int(row_stride), int(head_stride), _ptr(r), r.shape[0], float(scale),
                        _ptr(out), _ptr(lse))
    return out, lse


# -------------------------------------------------------- whole requests --

def decode_request(q_idx, w_idx, keys, ctx, n_cand, topk, q_attn_bits, scale, *,
                   pos2slot=None, hot_bits=None, pool_bits=None, k_cache_bits=None,
                   v_cache_bits=None, n_kv_heads=1, v_dim=512, row_stride=576,
                   head_stride=0):
    """One request of the whole decode step (every stage, in order).

    With a hot buffer (pos2slot given): hot_bits [S+topk, row] is updated in
    place with the gathered misses; pool_bits [L, row].  Without: attention
    reads k_cache_bits / v_cache_bits at the selected positions.
    Returns dict(cand, topk, topk_score, rows, n_miss, out, lse)."""
    q_idx, w_idx, keys = _c(q_idx, np.int8), _c(w_idx, np.int8), _c(keys, np.int8)
    qa = _c(q_attn_bits, np.uint16)
    h, d = q_idx.shape
    hq, dqk = qa.shape
    cand = np.empty(n_cand, np.int32)
    tk = np.empty(topk, np.int32)
    ts = np.empty(topk, np.int64)
    rows = np.empty(topk, np.int32)
    out = np.empty((hq, v_dim), np.float64)
    lse = np.empty(hq, np.float64)
    if pos2slot is not None:
        p2s = _c(pos2slot, np.int32)
        assert hot_bits.flags.c_contiguous and pool_bits.flags.c_contiguous
        # a row of the hot buffer and the pool is one latent row of row_stride
        # elements (the C side indexes both with it)
        assert hot_bits.shape[1] == row_stride and pool_bits.shape[1] == row_stride, \
            "hot/pool rows must be row_stride elements"
        hot_slots = hot_bits.shape[0] - topk
        kc = vc = None
    else:
        p2s, hot_slots = None, -1
        kc, vc = _c(k_cache_bits, np.uint16), _c(v_cache_bits, np.uint16)
    n_miss = lib().orc_decode_request(
        _ptr(q_idx), _ptr(w_idx), h, d, _ptr(keys), int(ctx), int(n_cand), int(topk),
        _ptr(p2s), int(hot_slots), _ptr(hot_bits), _ptr(pool_bits), _ptr(qa), hq,
        int(n_kv_heads), dqk, int(v_dim), _ptr(kc), _ptr(vc), int(row_stride),
        int(head_stride), float(scale), _ptr(cand), _ptr(tk), _ptr(ts), _ptr(rows),
        _ptr(out), _ptr(lse))
    return dict(cand=cand, topk=tk, topk_score=ts, rows=rows, n_miss=int(n_miss), out=out,
                lse=lse)


def prefill_row(q_row, w_row, keys, p: int, topk: int):
    """Top-k of one prefill query row at absolute position p (keys 0..p)."""
    q, w, k = _c(q_row, np.int8), _c(w_row, np.int8), _c(keys, np.int8)
    h, d = q.shape
    out = np.empty(topk, np.int32)
    sc = np.empty(topk, np.int64)
    lib().orc_prefill_row(_ptr(q), _ptr(w), h, d, _ptr(k), int(p), int(topk), _ptr(out),
                          _ptr(sc))
    return out, sc
