"""Pins for the CPU oracle: each oracle function is checked against something
other than itself -- hand-worked fixtures, closed forms, special cases that
reduce to a library routine (numpy floor division, numpy sort), and brute force
on tiny inputs written independently in numpy.  No GPU needed."""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _np_rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------- brute force --

def brute_scores(q, w, keys, coarse):
    """numpy: sum_h w_h * relu(q_h . key), key floor-divided by 16 if coarse."""
    k = keys.astype(np.int64)
    if coarse:
        k = np.floor_divide(k, 16)
    dots = q.astype(np.int64) @ k.T                  # [H, L]
    return (w.astype(np.int64)[:, None] * np.maximum(dots, 0)).sum(0)


def brute_select(score, pos, m):
    """numpy: lexsort by (score desc, pos asc), first m, ascending positions."""
    order = np.lexsort((pos, -score))
    keep = order[: min(m, len(score))]
    keep = keep[np.argsort(pos[keep], kind="stable")]
    return pos[keep], score[keep]


def brute_attention(q, k, v, scale):
    """numpy float64 softmax attention; q [Hq, dqk], k [n, dqk], v [n, dv]."""
    s = scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ v) / l, (m + np.log(l))[:, 0]


def bf16_bits(x):
    """float -> bfloat16 bits, round to nearest even (numpy, test-side)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_indexer(rng, H, D, L, lo=-127, hi=127):
    q = rng.integers(lo, hi + 1, size=(H, D)).astype(np.int8)
    w = rng.integers(1, 17, size=H).astype(np.int8)
    k = rng.integers(lo, hi + 1, size=(L, D)).astype(np.int8)
    return q, w, k


# ----------------------------------------------------------- A0: keys --

def test_coarse_value_exhaustive_matches_floor_division():
    for k in range(-128, 128):
        assert orc.coarse_value(k) == k // 16, k   # Python // is floor division


@pytest.mark.parametrize("k,expect", [(127, 7), (-127, -8), (100, 6), (-100, -7), (-1, -1),
                                      (15, 0), (16, 1), (-16, -1), (-17, -2), (-128, -8),
                                      (0, 0), (-33, -3)])
def test_coarse_value_reading(k, expect):
    assert orc.coarse_value(k) == expect


def test_pack_nibble_layout_by_hand():
    # element 2j in the low nibble, 2j+1 in the high nibble, two's complement
    k = np.array([[-16, 0, 0, -16, 127, -128, 16, 32]], dtype=np.int8)
    # pairs (-1,0) -> 0x0F; (0,-1) -> 0xF0; (7,-8) -> 0x87; (1,2) -> 0x21
    assert orc.pack_coarse(k).tolist() == [[0x0F, 0xF0, 0x87, 0x21]]


def test_pack_unpack_identity_all_values():
    vals = np.arange(-128, 128, dtype=np.int64)
    k = np.stack(np.meshgrid(vals, vals), -1).reshape(-1, 2).astype(np.int8)  # all pairs
    kc = orc.pack_coarse(k)
    back = orc.unpack_coarse(kc)
    assert np.array_equal(back.astype(np.int64), np.floor_divide(k.astype(np.int64), 16))


# ------------------------------------------- golden hand-worked example --

def test_hand_example_scores_and_selection():
    g = json.load(open(os.path.join(GOLD, "hand_indexer.json")))
    q = np.array(g["q"], np.int8)
    w = np.array(g["w"], np.int8)
    keys = np.array(g["keys"], np.int8)
    kc = orc.unpack_coarse(orc.pack_coarse(keys))
    assert kc.tolist() == g["coarse_keys"]
    assert orc.index_scores(q, w, keys, coarse=True).tolist() == g["coarse_scores"]
    assert orc.index_scores(q, w, keys, coarse=False).tolist() == g["fine_scores"]
    L = keys.shape[0]
    for case in g["cases"]:
        H = q.shape[0]
        qa = np.zeros((1, 8), np.uint16)
        kv = np.zeros((L, 8), np.uint16)
        r = orc.decode_request(q, w, keys, L, case["n_cand"], case["topk"], qa, 1.0,
                               k_cache_bits=kv, v_cache_bits=kv, n_kv_heads=1, v_dim=8,
                               row_stride=8, head_stride=0)
        assert r["cand"].tolist() == case["cand"], case
        assert r["topk"].tolist() == case["topk_pos"], case
        assert r["topk_score"].tolist() == case["topk_score"], case


def test_hand_example_attention():
    g = json.load(open(os.path.join(GOLD, "hand_attention.json")))
    q = bf16_bits(np.array(g["q"]))
    k = bf16_bits(np.array(g["k"]))
    v = bf16_bits(np.array(g["v"]))
    # K and V as separate caches, one kv head, head_dim 2
    out, lse = orc.attention(q, k.reshape(-1), v.reshape(-1), np.array([0, 1], np.int32),
                             g["scale"], 1, 2, 2, 0)
    np.testing.assert_allclose(out, np.array(g["out"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, np.array(g["lse"]), rtol=0, atol=1e-15)


# ------------------------------------------------ A1/A3: scoring pins --

@pytest.mark.parametrize("H,D,L,seed", [(1, 8, 20, 1), (4, 16, 37, 2), (3, 32, 64, 3),
                                        (8, 64, 50, 4)])
@pytest.mark.parametrize("coarse", [True, False])
def test_scores_brute_force(H, D, L, seed, coarse):
    q, w, k = rand_indexer(_np_rng(seed), H, D, L)
    assert np.array_equal(orc.index_scores(q, w, k, coarse), brute_scores(q, w, k, coarse))


def test_scores_negative_and_zero_weights_brute_force():
    rng = _np_rng(11)
    q, _, k = rand_indexer(rng, 5, 16, 40)
    w = np.array([-128, -3, 0, 5, 127], np.int8)
    for coarse in (True, False):
        assert np.array_equal(orc.index_scores(q, w, k, coarse), brute_scores(q, w, k, coarse))


def test_scores_one_hot_closed_form():
    # q[h] = 127 e_d for every head: score = (sum w) * max(0, 127 * key[d])
    rng = _np_rng(5)
    H, D, L, d = 4, 16, 64, 5
    _, w, k = rand_indexer(rng, H, D, L)
    q = np.zeros((H, D), np.int8)
    q[:, d] = 127
    sw = int(w.astype(np.int64).sum())
    kc = np.floor_divide(k[:, d].astype(np.int64), 16)
    expect_c = sw * np.maximum(0, 127 * kc)
    expect_f = sw * np.maximum(0, 127 * k[:, d].astype(np.int64))
    assert orc.index_scores(q, w, k, True).tolist() == expect_c.tolist()
    assert orc.index_scores(q, w, k, False).tolist() == expect_f.tolist()


def test_scores_single_head_unit_weight_is_relu_dot():
    rng = _np_rng(6)
    q, _, k = rand_indexer(rng, 1, 32, 50)
    w = np.ones(1, np.int8)
    expect = np.maximum(np.dot(k.astype(np.int64), q[0].astype(np.int64)), 0)
    assert np.array_equal(orc.index_scores(q, w, k, False), expect)


def test_scores_extreme_magnitude_int64():
    # every product at its extreme: 64 heads x 128 dims, w = 127
    H, D = 64, 128
    q = np.full((H, D), -127, np.int8)
    k = np.full((2, D), -127, np.int8)
    w = np.full(H, 127, np.int8)
    expect = H * 127 * (D * 127 * 127)
    assert orc.index_scores(q, w, k, False).tolist() == [expect, expect]
    assert expect > 2 ** 31    # exceeds int32: the oracle must carry int64


def test_scores_at_listed_positions():
    rng = _np_rng(7)
    q, w, k = rand_indexer(rng, 4, 16, 60)
    pos = np.array([59, 0, 17, -1, 3], np.int32)
    got = orc.index_scores_at(q, w, k, pos, coarse=False)
    full = brute_scores(q, w, k, False)
    assert got.tolist() == [full[59], full[0], full[17], 0, full[3]]


# -------------------------------------------------- A2/A4: selection --

@pytest.mark.parametrize("n,m,levels,seed", [(50, 10, 1000, 1), (50, 10, 3, 2), (200, 64, 5, 3),
                                             (30, 30, 4, 4), (30, 45, 4, 5), (1, 1, 2, 6),
                                             (100, 0, 2, 7)])
def test_select_brute_force_with_ties(n, m, levels, seed):
    rng = _np_rng(seed)
    score = rng.integers(-levels, levels, size=n).astype(np.int64)
    pos = rng.permutation(10 * n)[:n].astype(np.int32)
    got_p, got_s = orc.select_top(score, pos, m)
    exp_p, exp_s = brute_select(score, pos, m)
    assert got_p.tolist() == exp_p.tolist()
    assert got_s.tolist() == exp_s.tolist()


def test_select_all_equal_takes_lowest_positions():
    n, m = 100, 17
    got_p, _ = orc.select_top(np.full(n, 42, np.int64), np.arange(n, dtype=np.int32), m)
    assert got_p.tolist() == list(range(m))


def test_select_m_at_least_n_takes_everything():
    rng = _np_rng(9)
    s = rng.integers(0, 5, 20).astype(np.int64)
    got_p, _ = orc.select_top(s, np.arange(20, dtype=np.int32), 50)
    assert got_p.tolist() == list(range(20))


def test_full_candidates_equal_exact_topk():
    # with C = all tokens, coarse-to-fine must equal the exact top-k of fine scores
    rng = _np_rng(10)
    H, D, L, k = 4, 64, 300, 40
    q, w, keys = rand_indexer(rng, H, D, L)
    qa = np.zeros((1, 8), np.uint16)
    kv = np.zeros((L, 8), np.uint16)
    r = orc.decode_request(q, w, keys, L, L, k, qa, 1.0, k_cache_bits=kv, v_cache_bits=kv,
                           v_dim=8, row_stride=8)
    fine = brute_scores(q, w, keys, False)
    exp_p, exp_s = brute_select(fine, np.arange(L, dtype=np.int32), k)
    assert r["topk"].tolist() == exp_p.tolist()
    assert r["topk_score"].tolist() == exp_s.tolist()
    assert r["cand"].tolist() == list(range(L))


def test_coarse_to_fine_steps_brute_force():
    # stage by stage against numpy brute force, with C < L so the coarse pass matters
    rng = _np_rng(12)
    H, D, L, C, k = 4, 32, 500, 60, 20
    q, w, keys = rand_indexer(rng, H, D, L)
    qa = np.zeros((1, 8), np.uint16)
    kv = np.zeros((L, 8), np.uint16)
    r = orc.decode_request(q, w, keys, L, C, k, qa, 1.0, k_cache_bits=kv, v_cache_bits=kv,
                           v_dim=8, row_stride=8)
    cs = brute_scores(q, w, keys, True)
    cand, _ = brute_select(cs, np.arange(L, dtype=np.int32), C)
    assert r["cand"].tolist() == cand.tolist()
    fs = brute_scores(q, w, keys, False)[cand]
    top, top_s = brute_select(fs, cand, k)
    assert r["topk"].tolist() == top.tolist()
    assert r["topk_score"].tolist() == top_s.tolist()


def test_ctx_shorter_than_buffer_pads():
    rng = _np_rng(13)
    H, D, L = 2, 16, 40
    q, w, keys = rand_indexer(rng, H, D, L)
    qa = np.zeros((1, 8), np.uint16)
    kv = np.zeros((L, 8), np.uint16)
    r = orc.decode_request(q, w, keys, 7, 10, 12, qa, 1.0, k_cache_bits=kv, v_cache_bits=kv,
                           v_dim=8, row_stride=8)
    assert r["cand"].tolist()[:7] == list(range(7)) and r["cand"].tolist()[7:] == [-1] * 3
    assert r["topk"].tolist()[7:] == [-1] * 5
    assert sorted(r["topk"].tolist()[:7]) == list(range(7))


# -------------------------------------------------- A5/A6: hot buffer --

def test_hot_resolve_and_gather_brute_force():
    rng = _np_rng(14)
    L, S, row = 200, 16, 6
    sel = np.sort(rng.permutation(L)[:12]).astype(np.int32)
    pos2slot = np.full(L, -1, np.int32)
    resident = rng.permutation(L)[:S]
    pos2slot[resident] = rng.permutation(S)
    pool = rng.integers(0, 65535, size=(L, row)).astype(np.uint16)
    hot = np.zeros((S + len(sel), row), np.uint16)
    for t in resident:
        hot[pos2slot[t]] = pool[t]
    rows, miss = orc.hot_resolve(sel, pos2slot, S)
    exp_miss = [int(t) for t in sel if pos2slot[t] < 0]
    assert miss.tolist() == exp_miss
    j = 0
    for i, t in enumerate(sel):
        if pos2slot[t] >= 0:
            assert rows[i] == pos2slot[t]
        else:
            assert rows[i] == S + j
            j += 1
    orc.hot_gather(pool, miss, hot, S)
    for i, t in enumerate(sel):     # every resolved row holds the token's pool row
        assert np.array_equal(hot[rows[i]], pool[t])


# ------------------------------------------------------ A7/A8: attention --

def _rand_bits(rng, shape):
    return bf16_bits(rng.standard_normal(shape).astype(np.float32))


def test_attention_all_rows_equals_dense_mla():
    rng = _np_rng(20)
    n, hq, dqk, dv = 37, 16, 576, 512
    q = _rand_bits(rng, (hq, dqk))
    kv = _rand_bits(rng, (n, dqk))
    scale = 1 / math.sqrt(192)
    out, lse = orc.attention(q, kv.reshape(-1), kv.reshape(-1), np.arange(n, dtype=np.int32),
                             scale, 1, dv, dqk, 0)
    e_out, e_lse = brute_attention(bits_to_f64(q), bits_to_f64(kv), bits_to_f64(kv)[:, :dv],
                                   scale)
    np.testing.assert_allclose(out, e_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, e_lse, rtol=0, atol=1e-12)


def test_attention_gqa_head_mapping_dense():
    rng = _np_rng(21)
    n, hq, nkv, d = 25, 8, 2, 64
    q = _rand_bits(rng, (hq, d))
    K = _rand_bits(rng, (n, nkv, d))
    V = _rand_bits(rng, (n, nkv, d))
    rows = np.arange(n, dtype=np.int32)
    out, lse = orc.attention(q, K.reshape(-1), V.reshape(-1), rows, 0.125, nkv, d, nkv * d, d)
    for h in range(hq):
        g = h // (hq // nkv)
        e_out, e_lse = brute_attention(bits_to_f64(q[h:h + 1]), bits_to_f64(K[:, g]),
                                       bits_to_f64(V[:, g]), 0.125)
        np.testing.assert_allclose(out[h], e_out[0], atol=1e-12)
        np.testing.assert_allclose(lse[h], e_lse[0], atol=1e-12)


def test_attention_single_row_and_repeated_rows():
    rng = _np_rng(22)
    q = _rand_bits(rng, (4, 64))
    kv = _rand_bits(rng, (3, 64))
    s = 0.125 * (bits_to_f64(q) @ bits_to_f64(kv[1]))
    out, lse = orc.attention(q, kv.reshape(-1), kv.reshape(-1), np.array([1], np.int32), 0.125,
                             1, 64, 64, 0)
    np.testing.assert_array_equal(out, np.tile(bits_to_f64(kv[1]), (4, 1)))
    np.testing.assert_allclose(lse, s, atol=1e-14)
    out5, lse5 = orc.attention(q, kv.reshape(-1), kv.reshape(-1), np.full(5, 1, np.int32),
                               0.125, 1, 64, 64, 0)
    np.testing.assert_allclose(out5, out, atol=1e-15)
    np.testing.assert_allclose(lse5, s + math.log(5), atol=1e-13)


def test_attention_permutation_invariant_and_padding():
    rng = _np_rng(23)
    q = _rand_bits(rng, (4, 64))
    kv = _rand_bits(rng, (30, 64))
    rows = rng.permutation(30)[:12].astype(np.int32)
    a, la = orc.attention(q, kv.reshape(-1), kv.reshape(-1), rows, 0.3, 1, 32, 64, 0)
    b, lb = orc.attention(q, kv.reshape(-1), kv.reshape(-1),
                          np.concatenate([rows[::-1], [-1, -1]]).astype(np.int32), 0.3, 1, 32,
                          64, 0)
    np.testing.assert_allclose(a, b, atol=1e-13)
    np.testing.assert_allclose(la, lb, atol=1e-13)


def test_attention_no_rows():
    q = np.zeros((2, 8), np.uint16)
    out, lse = orc.attention(q, np.zeros(8, np.uint16), np.zeros(8, np.uint16),
                             np.array([-1, -1], np.int32), 1.0, 1, 8, 8, 0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# --------------------------------------------------- A9: prefill rows --

def test_prefill_row_brute_force_and_decode_equivalence():
    rng = _np_rng(30)
    H, D, L, k = 4, 32, 120, 16
    keys = rng.integers(-127, 128, size=(L, D)).astype(np.int8)
    for p in (0, 5, 15, 16, 77, 119):
        q = rng.integers(-127, 128, size=(H, D)).astype(np.int8)
        w = rng.integers(1, 17, size=H).astype(np.int8)
        got, got_s = orc.prefill_row(q, w, keys, p, k)
        fs = brute_scores(q, w, keys[: p + 1], False)
        exp_p, exp_s = brute_select(fs, np.arange(p + 1, dtype=np.int32), k)
        n = len(exp_p)
        assert got[:n].tolist() == exp_p.tolist() and got[n:].tolist() == [-1] * (k - n)
        assert got_s[:n].tolist() == exp_s.tolist()
        # the decode path with every token a candidate gives the same row
        qa = np.zeros((1, 8), np.uint16)
        kv = np.zeros((L, 8), np.uint16)
        r = orc.decode_request(q, w, keys, p + 1, p + 1, k, qa, 1.0, k_cache_bits=kv,
                               v_cache_bits=kv, v_dim=8, row_stride=8)
        assert r["topk"].tolist() == got.tolist()


# ------------------------------------------------- whole decode request --

def test_decode_request_with_hot_buffer_end_to_end():
    rng = _np_rng(40)
    H, D, L, C, k, S = 4, 32, 400, 64, 24, 32
    q, w, keys = rand_indexer(rng, H, D, L)
    hq, dqk, dv = 16, 576, 512
    qa = _rand_bits(rng, (hq, dqk))
    pool = _rand_bits(rng, (L, dqk))
    # selection computed independently (numpy), then the hot buffer is laid out from it
    cs = brute_scores(q, w, keys, True)
    cand, _ = brute_select(cs, np.arange(L, dtype=np.int32), C)
    top, top_s = brute_select(brute_scores(q, w, keys, False)[cand], cand, k)
    pos2slot = np.full(L, -1, np.int32)
    hits = top[: k - 5]
    pos2slot[hits] = np.arange(len(hits))
    hot = np.zeros((S + k, dqk), np.uint16)
    hot[: len(hits)] = pool[hits]
    r = orc.decode_request(q, w, keys, L, C, k, qa, 0.07, pos2slot=pos2slot, hot_bits=hot,
                           pool_bits=pool, v_dim=dv, row_stride=dqk)
    assert r["topk"].tolist() == top.tolist() and r["n_miss"] == 5
    e_out, e_lse = brute_attention(bits_to_f64(qa), bits_to_f64(pool[top]),
                                   bits_to_f64(pool[top])[:, :dv], 0.07)
    np.testing.assert_allclose(r["out"], e_out, atol=1e-12)
    np.testing.assert_allclose(r["lse"], e_lse, atol=1e-12)


# ------------------------------------------------------------ cache commit --
# Pins of orc_cache_commit (least-recently-used insertion of a step's misses,
# a reading: the pages name caches reused across steps but no policy).

def fresh_cache(n_slots, n_pos):
    return (np.full(n_pos, -1, np.int32), np.full(n_slots, -1, np.int32),
            np.zeros(n_slots, np.uint32))


def test_cache_commit_hand_example():
    # four slots holding positions 10..13, last used at steps 5, 2, 2, 7
    p2s, s2p, st = fresh_cache(4, 64)
    for s_, t in enumerate([10, 11, 12, 13]):
        p2s[t], s2p[s_] = s_, t
    st[:] = [5, 2, 2, 7]
    dst, n_ins = orc.cache_commit(np.array([11, 20, 13, 30, 40], np.int32), 4, 9, p2s, s2p, st)
    # hits 11 (slot 1) and 13 (slot 3); misses 20, 30, 40; the two slots not
    # hit (0 at step 5, 2 at step 2) are both victims, taken in slot order
    assert dst.tolist() == [1, 0, 3, 2, -1] and n_ins == 2
    assert s2p.tolist() == [20, 11, 30, 13]
    assert st.tolist() == [9, 9, 9, 9]
    assert p2s[10] == -1 and p2s[12] == -1 and p2s[20] == 0 and p2s[30] == 2 and p2s[40] == -1
    assert p2s[11] == 1 and p2s[13] == 3


def test_cache_commit_oldest_first_then_lowest_slot():
    # six slots, one miss at a time: the victim is always the slot with the
    # oldest stamp, the lowest index among equal stamps
    p2s, s2p, st = fresh_cache(6, 100)
    for s_ in range(6):
        p2s[50 + s_], s2p[s_] = s_, 50 + s_
    st[:] = [4, 1, 3, 1, 2, 9]
    expect = [1, 3, 4, 2, 0, 5]
    for k, e in enumerate(expect):
        dst, n_ins = orc.cache_commit(np.array([k], np.int32), 6, 10 + k, p2s, s2p, st)
        assert dst.tolist() == [e] and n_ins == 1


def test_cache_commit_fills_free_slots_in_order_and_padding_is_skipped():
    p2s, s2p, st = fresh_cache(8, 40)
    dst, n_ins = orc.cache_commit(np.array([3, -1, 7, 9, -1], np.int32), 8, 1, p2s, s2p, st)
    assert dst.tolist() == [0, -1, 1, 2, -1] and n_ins == 3
    assert s2p.tolist()[:3] == [3, 7, 9] and st.tolist() == [1, 1, 1, 0, 0, 0, 0, 0]


def test_cache_commit_more_misses_than_slots():
    p2s, s2p, st = fresh_cache(3, 40)
    dst, n_ins = orc.cache_commit(np.arange(5, 10, dtype=np.int32), 3, 1, p2s, s2p, st)
    assert dst.tolist() == [0, 1, 2, -1, -1] and n_ins == 3
    # next step: hits on 5 and 7 keep their slots; only slot 1 may be evicted
    dst, n_ins = orc.cache_commit(np.array([5, 7, 20, 21], np.int32), 3, 2, p2s, s2p, st)
    assert dst.tolist() == [0, 2, 1, -1] and n_ins == 1
    assert p2s[6] == -1 and s2p.tolist() == [5, 20, 7]


class ListLRU:
    """An independent model of the same policy: the resident positions kept
    in one recency list (least recent first).  After each step the slots the
    step used move to the most-recent end in ascending slot order (equal
    recency is broken by slot index); victims are the first entries of the
    list that the step did not hit."""

    def __init__(self, n_slots):
        self.order = list(range(n_slots))   # slots, least recent first
        self.slot_pos = [-1] * n_slots
        self.where = {}

    def step(self, entries):
        hit = sorted({self.where[t] for t in entries if t >= 0 and t in self.where})
        misses = [t for t in entries if t >= 0 and t not in self.where]
        free = [s for s in self.order if s not in set(hit)]
        vic = sorted(free[: len(misses)])
        dst = []
        j = 0
        for t in entries:
            if t < 0:
                dst.append(-1)
            elif t in self.where:
                dst.append(self.where[t])
            elif j < len(vic):
                v = vic[j]
                j += 1
                if self.slot_pos[v] >= 0:
                    del self.where[self.slot_pos[v]]
                self.slot_pos[v], self.where[t] = t, v
                dst.append(v)
            else:
                dst.append(-1)
        used = sorted(set(hit) | set(vic))
        self.order = [s for s in self.order if s not in set(used)] + used
        return dst


@pytest.mark.parametrize("n_slots,n_pos,n_entries,seed", [(16, 64, 12, 0), (64, 512, 40, 1),
                                                           (33, 200, 50, 2)])
def test_cache_commit_matches_recency_list_model(n_slots, n_pos, n_entries, seed):
    rng = np.random.default_rng(seed)
    p2s, s2p, st = fresh_cache(n_slots, n_pos)
    model = ListLRU(n_slots)
    hot = rng.choice(n_pos, size=n_pos // 4, replace=False)
    for now in range(1, 40):
        # a drifting working set: most entries from a hot set, some anywhere
        pick = np.where(rng.random(n_entries) < 0.7, rng.choice(hot, n_entries),
                        rng.integers(0, n_pos, n_entries))
        ent = np.unique(pick).astype(np.int32)
        pad = rng.integers(0, 3)
        ent = np.concatenate([ent, np.full(pad, -1, np.int32)])
        dst, n_ins = orc.cache_commit(ent, n_slots, now, p2s, s2p, st)
        assert dst.tolist() == model.step(ent.tolist()), now
        # the tables stay coherent
        occ = np.where(s2p >= 0)[0]
        assert (p2s[s2p[occ]] == occ).all()
        assert int((p2s >= 0).sum()) == len(occ)
        if now % 7 == 0:
            hot = rng.choice(n_pos, size=n_pos // 4, replace=False)
