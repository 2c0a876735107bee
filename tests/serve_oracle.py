"""The oracle's side of a serving loop, for the GPU tests: per request the
key store, the pool, the hot KV buffer and the indexer-key cache with their
tables, stepped by the oracle alongside the library's committing decode steps
and new-token appends, and compared with the library's results after every
step (bit for bit; attention within the output and log-sum-exp tolerances).

The cache policy is the oracle's least-recently-used commit (orc.cache_commit):
the step's candidates go through the key cache, its selection through the hot
buffer; a missed row moves into the victim slot the commit gives it, or stays
in the step's scratch rows when there is none."""
import numpy as np
import torch

from oracle import oracle as orc
from tests.gpu_common import np_, bits, oracle_cand, oracle_topk, assert_attention_close


def empty_tables(B, L, S):
    return (np.full((B, L), -1, np.int32), np.full((B, S), -1, np.int32),
            np.zeros((B, S), np.uint32))


class ServeShadow:
    """keys int8 [B, L, D], pool bf16 [B, L, row], q_attn bf16 [B, Hq, row]
    (CPU tensors, copied); ctx the valid lengths.  Both caches start empty."""

    def __init__(self, wl, keys, pool, q_attn, ctx):
        self.wl = wl
        B, L = keys.shape[0], keys.shape[1]
        D, S, SK, K, row = wl.idx_dim, wl.hot_slots, wl.key_slots, wl.topk, wl.qk_dim
        self.B, self.S, self.SK, self.K = B, S, SK, K
        self.keys = keys.detach().cpu().clone()
        self.pool = pool.detach().cpu().clone()
        self.q_attn = q_attn.detach().cpu()
        self.ctx = list(ctx)
        self.hot = np.zeros((B, S + K, row), np.uint16)
        self.p2s, self.s2p, self.st = empty_tables(B, L, S)
        self.kp2s, self.ks2p, self.kst = empty_tables(B, L, SK)
        self.kcache = np.zeros((B, SK, D), np.int8)
        self.hits = 0

    def step(self, step, out, lse, q, w, now, what=""):
        """Run the oracle's step of every request with indexer query q and
        weights w (CPU tensors) and stamp now; compare the library's step
        (already synchronised) and advance the shadow state."""
        wl, S, SK, C, K = self.wl, self.S, self.SK, self.wl.n_cand, self.K
        for b in range(self.B):
            tag = (what, b)
            qb, wb, kb = q[b].numpy(), w[b].numpy(), self.keys[b].numpy()
            cand = oracle_cand(qb, wb, kb, self.ctx[b], C)
            assert np_(step.cand)[b].tolist() == cand.tolist(), (tag, "cand")
            # key cache: the candidates' hits, then the misses moved in
            n_kmiss = int(((cand >= 0) & (self.kp2s[b][np.maximum(cand, 0)] < 0)).sum())
            assert int(np_(step.n_key_miss)[b]) == n_kmiss, (tag, "key misses")
            kdst, _ = orc.cache_commit(cand, SK, now, self.kp2s[b], self.ks2p[b], self.kst[b])
            for i, t in enumerate(cand):
                if t >= 0 and kdst[i] >= 0:
                    self.kcache[b, kdst[i]] = kb[t]
            tk, ts = oracle_topk(qb, wb, kb, cand, K)
            assert np_(step.topk)[b].tolist() == tk.tolist(), (tag, "topk")
            assert np_(step.topk_score)[b].tolist() == ts.tolist(), (tag, "scores")
            # hot buffer: resolve against the state before the commit
            hot_b = self.hot[b].copy()
            r = orc.decode_request(qb, wb, kb, self.ctx[b], C, K, bits(self.q_attn[b]), wl.scale,
                                   pos2slot=self.p2s[b].copy(), hot_bits=hot_b,
                                   pool_bits=bits(self.pool[b]))
            self.hits += int(((tk >= 0) & (self.p2s[b][np.maximum(tk, 0)] >= 0)).sum())
            dst, _ = orc.cache_commit(tk, S, now, self.p2s[b], self.s2p[b], self.st[b])
            rows = r["rows"].copy()
            j = 0
            for i, t in enumerate(tk):
                if t < 0:
                    continue
                if rows[i] >= S:               # a miss: into its slot, or scratch row S + j
                    if dst[i] >= 0:
                        rows[i] = dst[i]
                        self.hot[b, dst[i]] = bits(self.pool[b, t])
                    else:
                        self.hot[b, S + j] = bits(self.pool[b, t])
                    j += 1
            assert np_(step.rows)[b].tolist() == rows.tolist(), (tag, "rows")
            assert int(np_(step.n_miss)[b]) == r["n_miss"], (tag, "n_miss")
            assert_attention_close(out[b:b + 1], lse[b:b + 1], r["out"][None], r["lse"][None],
                                   "%s request %d" % (what, b))

    def check_state(self, hot, tables, ktables, kcache, what=""):
        """The library's caches (device tensors) against the shadow's: the
        resident rows of both caches and all six tables."""
        for dev, ref, name in ((tables, (self.p2s, self.s2p, self.st), "hot"),
                               (ktables, (self.kp2s, self.ks2p, self.kst), "keys")):
            p2s, s2p, st = dev
            assert np.array_equal(np_(p2s), ref[0]), (what, name, "pos2slot")
            assert np.array_equal(np_(s2p), ref[1]), (what, name, "slot2pos")
            assert np.array_equal(np_(st).view(np.uint32), ref[2]), (what, name, "stamps")
        assert np.array_equal(bits(hot)[:, :self.S], self.hot[:, :self.S]), (what, "hot rows")
        assert np.array_equal(np_(kcache), self.kcache), (what, "key cache rows")

    def append(self, new_k, new_kv):
        """The step's new token (CPU tensors [B, D] int8 and [B, row] bf16) at
        each request's end, unless the request is full."""
        L = self.keys.shape[1]
        for b in range(self.B):
            if self.ctx[b] < L:
                self.keys[b, self.ctx[b]] = new_k[b]
                self.pool[b, self.ctx[b]] = new_kv[b]
                self.ctx[b] += 1

    def check_stores(self, k8, pool, ctx_len, what=""):
        """The library's key store, pool and lengths against the shadow's."""
        assert np_(ctx_len).tolist() == self.ctx, (what, "ctx_len")
        assert torch.equal(k8.cpu(), self.keys), (what, "key store")
        assert torch.equal(pool.cpu().view(torch.int16), self.pool.view(torch.int16)), (what,
                                                                                         "pool")
