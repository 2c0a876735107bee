"""Shared helpers of the GPU parity tests: oracle-side reference results for
one request, tensor <-> numpy conversion, tolerances."""
import concurrent.futures
import os

import numpy as np
import torch

from oracle import oracle as orc

# bf16 output vs the double oracle, and fp32 log-sum-exp (natural log)
OUT_TOL = 2e-2
LSE_TOL = 1e-4


def np_(t):
    return t.detach().to("cpu").contiguous().numpy()


def bits(t):
    """bf16 tensor -> uint16 numpy bit patterns."""
    return np_(t.view(torch.int16)).view(np.uint16)


def bf16_to_f64(t):
    return t.detach().to("cpu", torch.float32).double().numpy()


def oracle_cand(q, w, keys, ctx, C):
    cs = orc.index_scores(q, w, keys, True, n_keys=ctx)
    p, _ = orc.select_top(cs, np.arange(ctx, dtype=np.int32), C)
    return orc.pad(p, C, -1)


def oracle_topk(q, w, keys, cand, K):
    valid = cand[cand >= 0]
    fs = orc.index_scores_at(q, w, keys, valid, False)
    p, s = orc.select_top(fs, valid, K)
    return orc.pad(p, K, -1), orc.pad(s, K, 0)


def poison_(t):
    if t.dtype in (torch.float32, torch.bfloat16):
        t.fill_(float("nan"))
    else:
        t.fill_(-7)
    return t


def assert_attention_close(out, lse, e_out, e_lse, what=""):
    o = bf16_to_f64(out)
    l_ = np_(lse).astype(np.float64)
    fin = np.isfinite(e_lse)
    assert np.array_equal(np.isfinite(l_), fin), what + ": -inf pattern of lse differs"
    if fin.any():
        err = np.abs(l_[fin] - e_lse[fin])
        assert (err <= LSE_TOL).all(), "%s: lse max abs err %.3g (tol %.3g)" % (
            what, err.max(), LSE_TOL)
    err_o = np.abs(o - e_out).max() if o.size else 0.0
    assert err_o <= OUT_TOL, "%s: out max abs err %.3g" % (what, err_o)
    return err_o


def parallel_map(fn, items, max_workers=16):
    """fn over items on a pool of host threads (the oracle's C calls release
    the interpreter lock), in item order; at most 16 threads, the host share
    of one GPU."""
    items = list(items)
    n = max(1, min(max_workers, os.cpu_count() or 1, len(items)))
    with concurrent.futures.ThreadPoolExecutor(n) as ex:
        return list(ex.map(fn, items))
