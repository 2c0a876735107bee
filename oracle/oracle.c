/*
 * Plain CPU oracle for one decode step of an indexer-driven top-k
 * sparse-attention layer, and for the multi-query prefill indexer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library; the two meet only in the seeded input generator.
 *
 * Style: single-threaded, plain loops, no intrinsics, no blocking, no fusion.
 * Integer work in int64_t, attention in double.  Every step is written in the
 * order the method states it, so it can be checked against the pages by eye.
 *
 * Sources (page title, section):
 *   [LS]  LeanSparse: Memory-Efficient Serving for Native Sparse-Attention
 *         LLMs (arXiv 2611.04671), Abstract -- decode runs coarse-to-fine
 *         indexing: it searches compact key representations first and fetches
 *         the original indexer keys only for the candidates it refines;
 *         prefill streams each layer's history through two reusable buffers.
 *   [XM]  XM-Sparse: Pushing the Throughput Frontier of Sparse Attention with
 *         Netpreme X-Mem (digest), section "hot buffer reduces reads but
 *         cannot replace the full history" -- a per-request hot KV buffer sits
 *         in HBM; after each step's selection only the selected rows that
 *         missed it are fetched from the full history; 4096-token buffer,
 *         2048 rows selected per step.
 *   [DSA] Related-papers list, abstract on dynamic sparse attention -- the
 *         attention reads only a top-k subset of the cached rows.
 *
 * Readings where the pages are silent:
 *   - indexer score of token t: sum over heads h of w[h]*max(0, q[h].k[t]),
 *     one int8 key per token shared by all heads;
 *   - the compact key is the arithmetic (floor) shift k >> 4, a signed
 *     nibble in [-8, 7]; the query stays int8 in the coarse pass;
 *   - ordering for every selection: score descending, then position
 *     ascending; selected positions are reported in ascending order;
 *   - attention: softmax(scale * q.K) V over the selected rows, with the
 *     log-sum-exp in natural log.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- keys -- */

/* Compact key value of one int8 indexer key element: floor(k / 16), i.e. an
 * arithmetic right shift by four bits.  Written as explicit floor division so
 * that no compiler- or sign-dependent shift semantics are involved.          */
int32_t orc_coarse_value(int32_t k)
{
    if (k >= 0)
        return k / 16;
    return -((-k + 15) / 16);
}

/* Storage form of the compact keys: two signed nibbles per byte, element 2j in
 * the low nibble and element 2j+1 in the high nibble (two's complement).
 * k: [n_rows][dim] int8, kc: [n_rows][dim/2] bytes.                          */
void orc_pack_coarse(const int8_t *k, uint8_t *kc, int64_t n_rows, int32_t dim)
{
    for (int64_t r = 0; r < n_rows; r++) {
        for (int32_t j = 0; j < dim / 2; j++) {
            int32_t lo = orc_coarse_value(k[r * dim + 2 * j]);
            int32_t hi = orc_coarse_value(k[r * dim + 2 * j + 1]);
            uint32_t lo_bits = (uint32_t)(lo + 16) % 16; /* two's complement nibble */
            uint32_t hi_bits = (uint32_t)(hi + 16) % 16;
            kc[r * (dim / 2) + j] = (uint8_t)(lo_bits + 16 * hi_bits);
        }
    }
}

/* Inverse of the storage form: nibble -> signed value in [-8, 7].            */
void orc_unpack_coarse(const uint8_t *kc, int8_t *out, int64_t n_rows, int32_t dim)
{
    for (int64_t r = 0; r < n_rows; r++) {
        for (int32_t j = 0; j < dim / 2; j++) {
            uint32_t byte = kc[r * (dim / 2) + j];
            int32_t lo = (int32_t)(byte % 16);
            int32_t hi = (int32_t)(byte / 16);
            if (lo >= 8) lo -= 16;
            if (hi >= 8) hi -= 16;
            out[r * dim + 2 * j] = (int8_t)lo;
            out[r * dim + 2 * j + 1] = (int8_t)hi;
        }
    }
}

/* ------------------------------------------------------------- scoring -- */

/* Indexer score of one key row against a query of n_heads x dim:
 *   sum_h w[h] * max(0, sum_d q[h][d] * key[d])
 * With coarse != 0 every key element is first replaced by its compact value
 * floor(key[d] / 16) -- the "compact representation" search of [LS].        */
static int64_t index_score_row(const int8_t *q, const int8_t *w, int32_t n_heads,
                               int32_t dim, const int8_t *key, int32_t coarse)
{
    int64_t total = 0;
    for (int32_t h = 0; h < n_heads; h++) {
        int64_t dot = 0;
        for (int32_t d = 0; d < dim; d++) {
            int64_t kv = coarse ? orc_coarse_value(key[d]) : key[d];
            dot += (int64_t)q[h * dim + d] * kv;
        }
        if (dot < 0)
            dot = 0;
        total += (int64_t)w[h] * dot;
    }
    return total;
}

/* Scores of the first n_keys rows of keys ([n_keys][dim] int8).             */
void orc_index_scores(const int8_t *q, const int8_t *w, int32_t n_heads, int32_t dim,
                      const int8_t *keys, int64_t n_keys, int32_t coarse, int64_t *out)
{
    for (int64_t t = 0; t < n_keys; t++)
        out[t] = index_score_row(q, w, n_heads, dim, keys + t * dim, coarse);
}

/* Scores of listed rows only (the refinement of [LS]: original int8 keys are
 * fetched for the candidates alone).  pos[i] < 0 marks an unused slot and
 * gets score 0.                                                             */
void orc_index_scores_at(const int8_t *q, const int8_t *w, int32_t n_heads, int32_t dim,
                         const int8_t *keys, const int32_t *pos, int64_t n,
                         int32_t coarse, int64_t *out)
{
    for (int64_t i = 0; i < n; i++) {
        if (pos[i] < 0) {
            out[i] = 0;
            continue;
        }
        out[i] = index_score_row(q, w, n_heads, dim, keys + (int64_t)pos[i] * dim, coarse);
    }
}

/* ----------------------------------------------------------- selection -- */

typedef struct {
    int64_t score;
    int32_t pos;
} scored_pos;

/* Order used by every selection: score descending, then position ascending. */
static int by_score_then_pos(const void *a, const void *b)
{
    const scored_pos *x = (const scored_pos *)a, *y = (const scored_pos *)b;
    if (x->score != y->score)
        return x->score > y->score ? -1 : 1;
    if (x->pos != y->pos)
        return x->pos < y->pos ? -1 : 1;
    return 0;
}

static int by_pos(const void *a, const void *b)
{
    const scored_pos *x = (const scored_pos *)a, *y = (const scored_pos *)b;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

/* Keep the m best of n scored positions: sort all n by (score desc, position
 * asc), take the first min(m, n), then report them by ascending position.
 * out_pos / out_score receive min(m, n) entries (out_score may be NULL).
 * Returns the number kept.                                                  */
int64_t orc_select_top(const int64_t *score, const int32_t *pos, int64_t n, int64_t m,
                       int32_t *out_pos, int64_t *out_score)
{
    scored_pos *all = (scored_pos *)malloc((size_t)(n > 0 ? n : 1) * sizeof(scored_pos));
    for (int64_t i = 0; i < n; i++) {
        all[i].score = score[i];
        all[i].pos = pos[i];
    }
    qsort(all, (size_t)n, sizeof(scored_pos), by_score_then_pos);
    int64_t kept = m < n ? m : n;
    if (kept < 0)
        kept = 0;
    qsort(all, (size_t)kept, sizeof(scored_pos), by_pos);
    for (int64_t i = 0; i < kept; i++) {
        out_pos[i] = all[i].pos;
        if (out_score)
            out_score[i] = all[i].score;
    }
    free(all);
    return kept;
}

/* ---------------------------------------------------------- hot buffer -- */

/* Resolve the selected positions (ascending, n_sel of them) against the
 * request's hot buffer [XM]: pos2slot[t] >= 0 means token t is resident in
 * that slot.  A hit reads its slot; the j-th miss (in ascending position
 * order) is assigned scratch row hot_slots + j and recorded in miss_pos.
 * Returns the miss count.                                                   */
int32_t orc_hot_resolve(const int32_t *sel, int32_t n_sel, const int32_t *pos2slot,
                        int32_t hot_slots, int32_t *rows, int32_t *miss_pos)
{
    int32_t n_miss = 0;
    for (int32_t i = 0; i < n_sel; i++) {
        int32_t slot = pos2slot[sel[i]];
        if (slot >= 0) {
            rows[i] = slot;
        } else {
            rows[i] = hot_slots + n_miss;
            miss_pos[n_miss] = sel[i];
            n_miss++;
        }
    }
    return n_miss;
}

/* ---------------------------------------------------------- cache commit --
 *
 * [LS] Abstract: the indexer-key cache and the KV cache are kept apart and
 * reused across generation steps; [XM] digest, hot buffer section: a step
 * fetches only the selected rows missing from the buffer.  Neither page
 * gives an insertion or eviction policy.  Reading (least recently used):
 *
 *   A cache of n_slots rows serves one request.  stamp[s] is the step that
 *   last used slot s (0: never), slot2pos[s] the position it holds (-1: free),
 *   pos2slot[t] the slot of position t (-1: absent).  One step uses the
 *   entries pos[0..n) (ascending positions, -1 = padding, skipped):
 *     1. an entry t with 0 <= pos2slot[t] < n_slots is a hit: its slot's
 *        stamp becomes now;
 *     2. an entry with pos2slot[t] < 0 is a miss; misses are numbered
 *        j = 0, 1, ... in entry order;
 *     3. victims: among the slots not hit in this step, the
 *        min(#misses, #slots not hit) smallest by (stamp ascending, slot
 *        ascending); they are then taken in ascending slot order;
 *     4. miss j (while victims remain) moves into victim v_j: the position
 *        the victim held (if any) loses its slot, pos2slot[t_j] = v_j,
 *        slot2pos[v_j] = t_j, stamp[v_j] = now.
 *   dst[i] is entry i's slot after the commit (hits: their slot; inserted
 *   misses: their victim; misses left out and padding: -1).  Entries whose
 *   pos2slot value lies at or beyond n_slots are neither hits nor misses.
 *   Returns the number of misses inserted.                                  */
typedef struct {
    uint32_t stamp;
    int32_t slot;
} stamped_slot;

static int by_stamp_then_slot(const void *a, const void *b)
{
    const stamped_slot *x = (const stamped_slot *)a, *y = (const stamped_slot *)b;
    if (x->stamp != y->stamp)
        return x->stamp < y->stamp ? -1 : 1;
    return (x->slot > y->slot) - (x->slot < y->slot);
}

static int by_int32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

int32_t orc_cache_commit(const int32_t *pos, int32_t n, int32_t n_slots, uint32_t now,
                         int32_t *pos2slot, int64_t n_pos, int32_t *slot2pos, uint32_t *stamp,
                         int32_t *dst)
{
    char *hit = (char *)calloc((size_t)n_slots + 1, 1);
    stamped_slot *order = (stamped_slot *)malloc(((size_t)n_slots + 1) * sizeof(stamped_slot));
    int32_t *victim = (int32_t *)malloc(((size_t)n_slots + 1) * sizeof(int32_t));
    char *miss = (char *)calloc((size_t)n + 1, 1);
    int32_t n_miss = 0, n_hit = 0, n_free = 0;

    /* 1. hits (and 2. the misses, marked from the same table state) */
    for (int32_t i = 0; i < n; i++) {
        dst[i] = -1;
        if (pos[i] < 0)
            continue;
        int32_t s = pos2slot[pos[i]];
        if (s >= 0 && s < n_slots) {
            dst[i] = s;
            if (!hit[s]) {
                hit[s] = 1;
                n_hit++;
            }
        } else if (s < 0) {
            miss[i] = 1;
            n_miss++;
        }
    }
    /* 3. victims: the oldest slots not hit, then in slot order */
    for (int32_t s = 0; s < n_slots; s++) {
        if (!hit[s]) {
            order[n_free].stamp = stamp[s];
            order[n_free].slot = s;
            n_free++;
        }
    }
    qsort(order, (size_t)n_free, sizeof(stamped_slot), by_stamp_then_slot);
    int32_t n_vic = n_miss < n_free ? n_miss : n_free;
    for (int32_t j = 0; j < n_vic; j++)
        victim[j] = order[j].slot;
    qsort(victim, (size_t)n_vic, sizeof(int32_t), by_int32);
    for (int32_t s = 0; s < n_slots; s++)
        if (hit[s])
            stamp[s] = now;
    /* 2 + 4. misses in entry order move into the victims */
    int32_t j = 0;
    for (int32_t i = 0; i < n && j < n_vic; i++) {
        if (!miss[i])
            continue;
        int32_t v = victim[j++];
        int32_t old = slot2pos[v];
        if (old >= 0 && old < n_pos)
            pos2slot[old] = -1;
        pos2slot[pos[i]] = v;
        slot2pos[v] = pos[i];
        stamp[v] = now;
        dst[i] = v;
    }
    free(hit);
    free(order);
    free(victim);
    free(miss);
    return n_vic;
}

/* Fetch the missed rows from the full-history pool into the hot buffer's
 * scratch rows: hot[hot_slots + j] := pool[miss_pos[j]] (a byte copy of
 * row_bytes bytes).                                                         */
void orc_hot_gather(const uint8_t *pool, int64_t row_bytes, const int32_t *miss_pos,
                    int32_t n_miss, uint8_t *hot, int32_t hot_slots)
{
    for (int32_t j = 0; j < n_miss; j++)
        memcpy(hot + (int64_t)(hot_slots + j) * row_bytes,
               pool + (int64_t)miss_pos[j] * row_bytes, (size_t)row_bytes);
}

/* ----------------------------------------------------------- attention -- */

/* bfloat16 bit pattern -> exact double.                                     */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Attention of one request over its selected rows [DSA], in double:
 *   s_i = scale * sum_d q[h][d] * K_i[d]
 *   o[h] = sum_i exp(s_i - m) V_i / sum_i exp(s_i - m),  lse[h] = m + ln l.
 * Row i of the selection is rows[i] (rows[i] < 0 ends the list).  The K/V
 * element (row r, kv head g, dim d) is at base[r*row_stride + g*head_stride
 * + d]; query head h reads kv head h / (n_q_heads / n_kv_heads).
 * For a latent (MLA-style) cache k_base == v_base and V is the first v_dim
 * elements of the same row.  No valid row: o = 0, lse = -inf.              */
void orc_attention(const uint16_t *q, int32_t n_q_heads, int32_t n_kv_heads, int32_t qk_dim,
                   int32_t v_dim, const uint16_t *k_base, const uint16_t *v_base,
                   int64_t row_stride, int64_t head_stride, const int32_t *rows, int32_t n_rows,
                   double scale, double *out, double *lse)
{
    int32_t group = n_q_heads / n_kv_heads;
    int32_t n_valid = 0;
    while (n_valid < n_rows && rows[n_valid] >= 0)
        n_valid++;
    double *s = (double *)malloc((size_t)(n_valid > 0 ? n_valid : 1) * sizeof(double));
    for (int32_t h = 0; h < n_q_heads; h++) {
        int32_t g = h / group;
        double m = -INFINITY;
        for (int32_t i = 0; i < n_valid; i++) {
            const uint16_t *krow = k_base + (int64_t)rows[i] * row_stride + (int64_t)g * head_stride;
            double dot = 0.0;
            for (int32_t d = 0; d < qk_dim; d++)
                dot += bf16_to_double(q[(int64_t)h * qk_dim + d]) * bf16_to_double(krow[d]);
            s[i] = scale * dot;
            if (s[i] > m)
                m = s[i];
        }
        double l = 0.0;
        for (int32_t i = 0; i < n_valid; i++)
            l += exp(s[i] - m);
        for (int32_t d = 0; d < v_dim; d++) {
            double acc = 0.0;
            for (int32_t i = 0; i < n_valid; i++) {
                const uint16_t *vrow = v_base + (int64_t)rows[i] * row_stride + (int64_t)g * head_stride;
                acc += exp(s[i] - m) * bf16_to_double(vrow[d]);
            }
            out[(int64_t)h * v_dim + d] = n_valid > 0 ? acc / l : 0.0;
        }
        lse[h] = n_valid > 0 ? m + log(l) : -INFINITY;
    }
    free(s);
}

/* ------------------------------------------------------ whole requests -- */

/* One request of the decode step, every stage in order (used for the CPU
 * baseline timing and for end-to-end checks):
 *   1. coarse score of every cached token from its compact key       [LS]
 *   2. keep the n_cand best as candidates                            [LS]
 *   3. fine score of the candidates from their original int8 keys    [LS]
 *   4. keep the topk best of the candidates                          [LS][XM]
 *   5. resolve against the hot buffer, copy misses from the pool     [XM]
 *   6. attention over the selected rows (MLA layout, k == v base)    [DSA]
 * With hot_slots < 0 there is no hot buffer and step 6 reads rows of
 * k_cache/v_cache directly at the selected positions.
 * Outputs: cand [n_cand] (pad -1), topk [topk] (pad -1), topk_score,
 * rows [topk] (pad -1), out [Hq][v_dim], lse [Hq]; returns n_miss.          */
int32_t orc_decode_request(const int8_t *q_idx, const int8_t *w_idx, int32_t n_heads,
                           int32_t dim, const int8_t *keys, int32_t ctx, int32_t n_cand,
                           int32_t topk, const int32_t *pos2slot, int32_t hot_slots,
                           uint8_t *hot, const uint8_t *pool, const uint16_t *q_attn,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t qk_dim,
                           int32_t v_dim, const uint16_t *k_cache, const uint16_t *v_cache,
                           int64_t row_stride, int64_t head_stride, double scale,
                           int32_t *cand, int32_t *topk_pos, int64_t *topk_score,
                           int32_t *rows, double *out, double *lse)
{
    int64_t *cs = (int64_t *)malloc((size_t)(ctx > 0 ? ctx : 1) * sizeof(int64_t));
    int32_t *all_pos = (int32_t *)malloc((size_t)(ctx > 0 ? ctx : 1) * sizeof(int32_t));
    int64_t *fs = (int64_t *)malloc((size_t)(n_cand > 0 ? n_cand : 1) * sizeof(int64_t));
    int32_t *miss_pos = (int32_t *)malloc((size_t)(topk > 0 ? topk : 1) * sizeof(int32_t));

    orc_index_scores(q_idx, w_idx, n_heads, dim, keys, ctx, 1, cs);
    for (int32_t t = 0; t < ctx; t++)
        all_pos[t] = t;
    int64_t nc = orc_select_top(cs, all_pos, ctx, n_cand, cand, NULL);
    for (int64_t i = nc; i < n_cand; i++)
        cand[i] = -1;

    orc_index_scores_at(q_idx, w_idx, n_heads, dim, keys, cand, nc, 0, fs);
    int64_t nk = orc_select_top(fs, cand, nc, topk, topk_pos, topk_score);
    for (int64_t i = nk; i < topk; i++) {
        topk_pos[i] = -1;
        topk_score[i] = 0;
    }

    int32_t n_miss = 0;
    const uint16_t *kb = k_cache, *vb = v_cache;
    if (hot_slots >= 0) {
        n_miss = orc_hot_resolve(topk_pos, (int32_t)nk, pos2slot, hot_slots, rows, miss_pos);
        orc_hot_gather(pool, row_stride * 2, miss_pos, n_miss, hot, hot_slots);
        kb = (const uint16_t *)hot;
        vb = (const uint16_t *)hot;
    } else {
        for (int64_t i = 0; i < nk; i++)
            rows[i] = topk_pos[i];
    }
    for (int64_t i = nk; i < topk; i++)
        rows[i] = -1;

    orc_attention(q_attn, n_q_heads, n_kv_heads, qk_dim, v_dim, kb, vb, row_stride,
                  head_stride, rows, topk, scale, out, lse);
    free(cs);
    free(all_pos);
    free(fs);
    free(miss_pos);
    return n_miss;
}

/* Prefill-chunk indexer row [LS]: query row i sits at absolute position p and
 * sees keys 0..p (causal).  Its fine scores use its own weights; it keeps its
 * topk best under the same ordering.  Returns the number kept; out is padded
 * with -1 to topk.                                                          */
int64_t orc_prefill_row(const int8_t *q_row, const int8_t *w_row, int32_t n_heads, int32_t dim,
                        const int8_t *keys, int32_t p, int32_t topk, int32_t *out,
                        int64_t *out_score)
{
    int64_t n = (int64_t)p + 1;
    int64_t *sc = (int64_t *)malloc((size_t)n * sizeof(int64_t));
    int32_t *ps = (int32_t *)malloc((size_t)n * sizeof(int32_t));
    orc_index_scores(q_row, w_row, n_heads, dim, keys, n, 0, sc);
    for (int64_t t = 0; t < n; t++)
        ps[t] = (int32_t)t;
    int64_t kept = orc_select_top(sc, ps, n, topk, out, out_score);
    for (int64_t i = kept; i < topk; i++) {
        out[i] = -1;
        if (out_score)
            out_score[i] = 0;
    }
    free(sc);
    free(ps);
    return kept;
}
