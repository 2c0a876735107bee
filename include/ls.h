/*
 * ls.h -- C-ABI of the MI355X (gfx950) sparse-decode library libls.so.
 *
 * One decode step of an indexer-driven top-k sparse-attention layer, in four
 * stages, plus the multi-query prefill indexer:
 *
 *   1. coarse-to-fine indexer: score every cached token from compact 4-bit
 *      keys, keep n_cand candidates, re-score only those with their original
 *      int8 indexer keys.  [LeanSparse (arXiv 2611.04671), Abstract: decode
 *      searches compact representations and fetches the original indexer keys
 *      only for candidate refinement.]
 *   2. keep the topk best candidates.  [same Abstract; XM-Sparse digest,
 *      section on the hot buffer: 2048 rows selected per step.]
 *   3. resolve each selected token against the request's hot KV buffer and
 *      copy the misses from the full-history pool.  [XM-Sparse: Pushing the
 *      Throughput Frontier of Sparse Attention with Netpreme X-Mem (digest),
 *      section "hot buffer reduces reads but cannot replace the full
 *      history": only selected rows that missed the HBM hot buffer are
 *      fetched; 4096-token hot buffer per request and layer.]
 *   4. attention over the selected rows, split over the row list and merged
 *      by a combine pass.  [related-papers list, dynamic sparse attention
 *      abstract: each query reads only a top-k subset of the cached rows.]
 *   prefill: per query row of a prefill chunk, the causal top-k of the fine
 *      indexer score, with the layer's key history streamed through two
 *      reusable device buffers.  [LeanSparse Abstract: prefill streams layer
 *      histories through two reusable GPU buffers, overlapping the next
 *      layer's load with the current computation.]
 *
 * Definitions used throughout (readings where the pages give no formula):
 *   indexer score   s(t) = sum_h w[h] * max(0, sum_d q[h][d] * key[t][d]),
 *                   one int8 key row per token shared by all heads;
 *                   computed exactly (int32 per head, int64 across heads).
 *   compact key     kc = floor(k / 16) (arithmetic shift), a signed nibble;
 *                   stored two per byte, element 2j in the low nibble.
 *   selection order score descending, then position ascending; every index
 *                   output lists the kept positions in ascending order and
 *                   pads the rest with -1.
 *   attention       o[h] = softmax_i(scale * q[h].K_i) V_i over the selected
 *                   rows; lse[h] = natural-log log-sum-exp of the scaled
 *                   scores; no valid row gives o = 0, lse = -inf.
 *
 * Conventions for every call:
 *   - Ownership: the caller allocates and owns every buffer.  Entry points
 *     never allocate or free device memory.  Scratch space is a caller-owned
 *     workspace of ls_workspace_size() bytes that must be cleared once with
 *     ls_workspace_init() before its first use; every call leaves it cleared
 *     again for the next call.  Two calls that may run at the same time need
 *     two workspaces.
 *   - Asynchrony: calls only enqueue work on the given stream (NULL = the
 *     default stream) and return without waiting.  Device faults surface at
 *     the caller's next synchronisation.
 *   - Errors: every entry point returns LS_OK or a negative code.  Arguments
 *     are validated on the host before anything is enqueued; on failure
 *     nothing is enqueued.  ls_last_error() gives a message for the calling
 *     thread, ls_last_hip_error() the last HIP status.  No C++ exception
 *     crosses this interface.
 *   - Layout: dense row-major arrays, one block of max_ctx tokens per request.
 *     ctx_len[b] (device int32) is the number of valid tokens of request b;
 *     values are clamped to [0, max_ctx] on the device.  Pointers to int8 /
 *     uint8 / bf16 tensors must be 16-byte aligned.
 *   - Pointers named *_dev are device memory (or pinned host memory mapped
 *     for the device where stated); descriptors are host memory.
 */
#ifndef LS_H
#define LS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same handle types as the HIP runtime's hipStream_t / hipEvent_t. */
typedef struct ihipStream_t *ls_stream_t;
typedef struct ihipEvent_t *ls_event_t;

#define LS_ABI_VERSION 5

enum {
    LS_OK = 0,
    LS_E_ARG = -1,         /* null pointer, bad size or misaligned pointer   */
    LS_E_UNSUPPORTED = -2, /* valid request that no kernel here implements   */
    LS_E_WORKSPACE = -3,   /* workspace missing or smaller than required     */
    LS_E_HIP = -4          /* HIP runtime or launch error                    */
};

/* Operation ids for ls_workspace_size. */
enum {
    LS_OP_COARSE = 1,  /* desc: ls_idx_desc     */
    LS_OP_REFINE = 2,  /* desc: ls_idx_desc     */
    LS_OP_HOT = 3,     /* desc: ls_hot_desc     */
    LS_OP_ATTN = 4,    /* desc: ls_attn_desc    */
    LS_OP_STEP = 5,    /* desc: ls_step_desc    */
    LS_OP_PREFILL = 6  /* desc: ls_prefill_desc */
};

/* Indexer shapes.  n_heads in [1, 64]; head_dim 64 or 128; n_cand >= 1;
 * topk >= 1 (topk > n_cand is allowed and pads); max_ctx in [1, 2^28).
 *
 * Where the original int8 keys live (the refinement reads only the
 * candidates' rows of them):
 *   keys_on_host = 0: k8 [B, max_ctx, D] is device memory;
 *   keys_on_host = 1: k8 is pinned, device-mapped host memory, read over
 *     PCIe, so the full key history takes no HBM (only the compact keys
 *     stay on the GPU).
 *   key_slots > 0 adds a per-request indexer-key cache in device memory:
 *     kcache [B, key_slots, D] int8 with kpos2slot [B, max_ctx] int32 (the
 *     cache row of token t, -1 if absent; values outside [0, key_slots)
 *     count as absent).  A candidate whose key is cached is read from the
 *     cache and its k8 row is not touched.  The caller keeps the cache
 *     coherent with k8 (a cached row must equal the token's key); the
 *     library only reads it.  key_slots = 0: no cache, both pointers may be
 *     NULL.  key_slots <= 2^24.
 * [LeanSparse Abstract: the original indexer keys are kept off the GPU,
 *  fetched only for candidate refinement, and held in an indexer-key cache
 *  of their own that is reused across generation steps.]                    */
typedef struct {
    int32_t batch, max_ctx, n_heads, head_dim, n_cand, topk;
    int32_t keys_on_host, key_slots;
} ls_idx_desc;

/* Hot KV buffer of one layer.  Each request owns hot_slots resident rows
 * followed by topk scratch rows that receive the step's misses; a row is
 * row_elems bf16 values (a multiple of 8, with topk * row_elems * 2 bytes
 * below 2^32, else LS_E_UNSUPPORTED).  pool_on_host = 1 means the pool is
 * pinned host memory that the device reads over PCIe.                       */
typedef struct {
    int32_t batch, max_ctx, topk, hot_slots, row_elems, pool_on_host;
} ls_hot_desc;

/* Sparse decode attention.  One query token per request; n_q_heads query
 * heads share n_kv_heads kv heads (query head h reads kv head
 * h / (n_q_heads / n_kv_heads)).  The K/V element (request b, row r, kv head
 * g, dim d) is at base[(b * kv_rows_per_req + r) * kv_row_stride
 * + g * kv_head_stride + d].  For a latent (MLA-style) cache pass the same
 * base for K and V: V is then the first v_dim elements of the K row.
 * n_splits: number of row splits per request (0 = chosen by the library;
 * the latent-layout kernel raises it so that no split exceeds 1024 rows).
 * qk_dim is a multiple of 8; outside the latent layout (576 / 512, one kv
 * head) v_dim and both strides must be multiples of 8 too and topk at most
 * 8192, else LS_E_UNSUPPORTED.                                              */
typedef struct {
    int32_t batch, n_q_heads, n_kv_heads, qk_dim, v_dim, topk;
    int64_t kv_rows_per_req, kv_row_stride, kv_head_stride;
    float scale;
    int32_t n_splits;
} ls_attn_desc;

/* Cache commit of a step: the caches keep what the step used, so that the
 * next steps reuse it.  [LeanSparse Abstract: the indexer-key cache and the
 * KV cache are separate and reused across generation steps; XM-Sparse
 * digest, hot buffer section: only the selected rows missing from the
 * buffer are fetched.]  The pages give no policy; this one is least
 * recently used (see ls_cache_commit):
 *   hot = 1: the step's KV misses move into victim slots of the hot buffer
 *     (the gather writes each row straight into its slot, rows[] names the
 *     slot, pos2slot / slot2pos / stamp are updated); misses beyond the
 *     free slots stay in the scratch rows, uncached.  Needs use_hot = 1,
 *     hot_slots in [1, 16384], topk <= 16384.
 *   keys = 1: the step's candidates missing from the key cache move into
 *     victim rows of it (the refinement copies each key row it reads from
 *     k8 into its row; kpos2slot / kslot2pos / kstamp are updated).  Needs
 *     key_slots in [1, 16384], n_cand <= 16384.
 *   now: this step's stamp, below 2^32 - 1 and above every stamp already
 *     in the tables (a step counter starting at 1 over zeroed stamps).  With
 *     ls_step_io.now_dev set, the stamp is read from that device word
 *     instead, when the kernels run: a step captured once in a graph then
 *     stamps each replay with the counter's current value (the caller
 *     advances it between replays, for example inside the same graph).
 * Without commit (both 0) the step only reads the caches and is
 * idempotent.                                                               */
typedef struct {
    int32_t hot, keys;
    uint32_t now;
} ls_commit_desc;

/* Whole step.  With use_hot = 1 attention reads the hot buffer (MLA latent
 * rows, k_base = v_base = hot_kv); with use_hot = 0 it reads k_cache /
 * v_cache at the selected positions.                                        */
typedef struct {
    ls_idx_desc idx;
    ls_hot_desc hot;
    ls_attn_desc attn;
    int32_t use_hot;
    ls_commit_desc commit;
} ls_step_desc;

/* Number of stage events ls_decode_step records when given an event array:
 * [0] start, [1] after coarse scoring, [2] after candidate selection,
 * [3] after refinement + top-k (+ hot resolve), [4] after the miss gather,
 * [5] after the attention kernel, [6] after the combine pass (end).  A NULL
 * entry is skipped (each recorded event costs the stream a few
 * microseconds, so a caller that times one stage records only its two).
 * [0] and [1] given together are recorded by the coarse kernel's launch at
 * the kernel's own start and end, so their interval is that kernel alone.  */
#define LS_STEP_EVENTS 7

/* Device pointers of one step (see the individual stages for shapes). */
typedef struct {
    const int8_t *q_idx_dev;    /* [B, H, D] int8 indexer query              */
    const int8_t *w_idx_dev;    /* [B, H] int8 per-head weights              */
    const uint8_t *kc_dev;      /* [B, max_ctx, D/2] packed compact keys     */
    const int8_t *k8_dev;       /* [B, max_ctx, D] original int8 keys        */
    int32_t *kpos2slot_dev;     /* [B, max_ctx] key-cache row or -1 (nullable;
                                   written by commit.keys)                   */
    int8_t *kcache_dev;         /* [B, key_slots, D] key cache (nullable;
                                   written by commit.keys)                   */
    const int32_t *ctx_len_dev; /* [B] valid tokens per request              */
    int32_t *cand_dev;          /* out [B, n_cand] candidates                */
    int32_t *topk_dev;          /* out [B, topk] selected positions          */
    int64_t *topk_score_dev;    /* out [B, topk] their fine scores (nullable)*/
    int32_t *pos2slot_dev;      /* [B, max_ctx] hot slot of a token or -1
                                   (written by commit.hot)                   */
    void *hot_kv_dev;           /* [B, hot_slots + topk, row] bf16 (in/out)  */
    const void *pool_kv_dev;    /* [B, max_ctx, row] bf16 full history       */
    int32_t *rows_dev;          /* out [B, topk] row read for each selected  */
    int32_t *n_miss_dev;        /* out [B] misses fetched                    */
    const void *q_attn_dev;     /* [B, Hq, qk_dim] bf16 attention query      */
    const void *k_cache_dev;    /* use_hot = 0 only: K cache                 */
    const void *v_cache_dev;    /* use_hot = 0 only: V cache                 */
    void *out_dev;              /* out [B, Hq, v_dim] bf16                   */
    float *lse_dev;             /* out [B, Hq] fp32                          */
    ls_event_t *stage_events;   /* nullable: LS_STEP_EVENTS events to record */
    int32_t *slot2pos_dev;      /* [B, hot_slots] token of each slot or -1,
                                   in/out (commit.hot; else nullable)        */
    uint32_t *stamp_dev;        /* [B, hot_slots] step that last used each
                                   slot, in/out (commit.hot; else nullable)  */
    int32_t *kslot2pos_dev;     /* [B, key_slots] (commit.keys; else nullable)*/
    uint32_t *kstamp_dev;       /* [B, key_slots] (commit.keys; else nullable)*/
    int32_t *n_key_miss_dev;    /* out [B] (nullable; written with commit.keys):
                                   candidates whose key was read from k8     */
    const uint32_t *now_dev;    /* nullable: the commit's stamp, read on the
                                   device (see ls_commit_desc)               */
} ls_step_io;

/* Prefill chunk: n_query query tokens at absolute positions
 * q_pos0 .. q_pos0 + n_query - 1 over a history of max_ctx keys (causal:
 * query i sees keys 0 .. q_pos0 + i).  max_ctx * head_dim below 2^31 (else
 * LS_E_UNSUPPORTED).                                                       */
typedef struct {
    int32_t n_query, max_ctx, q_pos0, n_heads, head_dim, topk;
} ls_prefill_desc;

/* ------------------------------------------------------------ library -- */

int32_t ls_abi_version(void);
const char *ls_last_error(void);
int32_t ls_last_hip_error(void);

/* Workspace bytes needed by operation op for the shapes in desc (0 on a bad
 * descriptor, with the reason in ls_last_error()).                          */
size_t ls_workspace_size(int32_t op, const void *desc);

/* Clear a workspace before its first use (enqueues a fill kernel).          */
int ls_workspace_init(void *ws_dev, size_t ws_bytes, ls_stream_t stream);

/* -------------------------------------------------------------- stages -- */

/* Compact keys for storage: kc[r][j] packs floor(k[r][2j]/16) (low nibble)
 * and floor(k[r][2j+1]/16) (high nibble).  k8: [n_rows, dim] int8,
 * kc: [n_rows, dim/2]; dim even.  Runs when keys are appended, outside the
 * decode step.  [LeanSparse Abstract: compact representations.]             */
int ls_pack_coarse(const int8_t *k8_dev, uint8_t *kc_dev, int64_t n_rows, int32_t dim,
                   ls_stream_t stream);

/* Stage 1a: coarse scores of every valid token from the compact keys, then
 * the n_cand best under the selection order.  q: [B,H,D], w: [B,H],
 * kc: [B,max_ctx,D/2].  cand: out [B,n_cand] int32, ascending, -1 padded
 * (every valid token is a candidate when ctx_len <= n_cand).
 * [LeanSparse Abstract: coarse-to-fine indexing.]                           */
int ls_index_coarse(const ls_idx_desc *desc, const int8_t *q_dev, const int8_t *w_dev,
                    const uint8_t *kc_dev, const int32_t *ctx_len_dev, int32_t *cand_dev,
                    void *ws_dev, size_t ws_bytes, ls_stream_t stream);

/* Stage 1b + 2: exact scores of the candidates from their original int8 keys
 * k8 [B,max_ctx,D] (or the key cache, see ls_idx_desc), then the topk best.
 * cand as produced by ls_index_coarse (ascending, -1 padded).  topk: out
 * [B,topk] ascending, -1 padded; topk_score: out [B,topk] int64 (nullable;
 * 0 in padded slots).  kpos2slot / kcache: required iff desc->key_slots > 0.
 * [LeanSparse Abstract: original keys fetched only for refinement.]         */
int ls_refine_topk(const ls_idx_desc *desc, const int8_t *q_dev, const int8_t *w_dev,
                   const int8_t *k8_dev, const int32_t *kpos2slot_dev, const int8_t *kcache_dev,
                   const int32_t *cand_dev, const int32_t *ctx_len_dev, int32_t *topk_dev,
                   int64_t *topk_score_dev, void *ws_dev, size_t ws_bytes, ls_stream_t stream);

/* Stage 3: resolve the selected positions topk [B,topk] against
 * pos2slot [B,max_ctx] (slot of a resident token, -1 if absent).  A hit reads
 * slot pos2slot[t]; the j-th miss of a request (ascending position order) is
 * copied from pool [B,max_ctx,row] into scratch row hot_slots + j of hot_kv
 * [B,hot_slots+topk,row].  rows: out [B,topk] (the hot_kv row of every
 * selected token, -1 for padding); n_miss: out [B].  The pool may be pinned
 * host memory (pool_on_host = 1).  [XM-Sparse digest, hot buffer section.] */
int ls_hot_gather(const ls_hot_desc *desc, const int32_t *topk_dev, const int32_t *pos2slot_dev,
                  void *hot_kv_dev, const void *pool_kv_dev, int32_t *rows_dev,
                  int32_t *n_miss_dev, void *ws_dev, size_t ws_bytes, ls_stream_t stream);

/* Stage 4: attention of q [B,Hq,qk_dim] bf16 over the rows listed in
 * rows [B,topk] of the K/V bases described in desc; -1, and any id outside
 * [0, kv_rows_per_req), is padding and is skipped.  out: [B,Hq,v_dim] bf16
 * (round to nearest even), lse: [B,Hq] fp32 (-inf and a zero output when a
 * request lists no row).
 * [related-papers list, dynamic sparse attention abstract.]                 */
int ls_sparse_attn_decode(const ls_attn_desc *desc, const void *q_dev, const void *k_base_dev,
                          const void *v_base_dev, const int32_t *rows_dev, void *out_dev,
                          float *lse_dev, void *ws_dev, size_t ws_bytes, ls_stream_t stream);

/* The whole decode step, stages 1-4 in order on one stream.                 */
int ls_decode_step(const ls_step_desc *desc, const ls_step_io *io, void *ws_dev,
                   size_t ws_bytes, ls_stream_t stream);

/* The same step without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Its scratch is a static 128 MiB array
 * that the library holds on each device it runs on until the process ends;
 * a step whose workspace (ls_workspace_size(LS_OP_STEP, desc)) exceeds it is
 * rejected with LS_E_UNSUPPORTED before anything is enqueued.  Each call
 * first clears the part of the scratch that must start at zero (one small
 * fill kernel), then runs exactly the kernels of ls_decode_step.  Every call
 * on a device shares that device's scratch: calls that overlap on one device
 * (two streams, or two threads) race and must not be issued.  Nothing here
 * allocates or frees memory.                                                */
int ls_decode_step_noalloc(const ls_step_desc *desc, const ls_step_io *io, ls_stream_t stream);

/* One least-recently-used commit per request into a cache of n_slots rows
 * (the hot KV buffer or the indexer-key cache; the step runs the same
 * commit when ls_commit_desc asks for it).  entries [B, n]: the positions
 * the step used, ascending and distinct, -1 padded.  Tables, updated in place:
 * pos2slot [B, max_ctx] (slot of a token or -1), slot2pos [B, n_slots]
 * (token of a slot or -1), stamp [B, n_slots] (step that last used the
 * slot, 0 = never).
 *   1. an entry with pos2slot in [0, n_slots) is a hit: stamp := now;
 *   2. an entry with pos2slot < 0 is a miss; misses are numbered in entry
 *      order;
 *   3. victims: of the slots not hit, the min(#misses, #not hit) with the
 *      smallest (stamp, slot index), taken in ascending slot order;
 *   4. miss j moves into victim j: the token the victim held loses its slot,
 *      pos2slot / slot2pos updated, stamp := now.
 * dst: out [B, n], each entry's slot after the commit (-1: padding or a
 * miss left out).  n_inserted: out [B] (nullable).  n_slots and n in
 * [1, 16384]; now < 2^32 - 1.  Moving the rows' data is the caller's (the
 * decode step does it for both caches).  Tables must be coherent
 * (pos2slot[slot2pos[s]] == s); positions must be below max_ctx.
 * [Reading of LeanSparse Abstract, caches reused across steps.]            */
int ls_cache_commit(int32_t batch, int32_t max_ctx, int32_t n_slots, int32_t n, uint32_t now,
                    const int32_t *entries_dev, int32_t *pos2slot_dev, int32_t *slot2pos_dev,
                    uint32_t *stamp_dev, int32_t *dst_dev, int32_t *n_inserted_dev,
                    ls_stream_t stream);

/* New-token append (once per generated token and layer): the token of
 * request b goes to position ctx_len[b] when that is below max_ctx (a full
 * request is left unchanged): new_k8 [B, head_dim] int8 into k8 (device, or
 * pinned host with keys_on_host = 1), its compact form into kc, and, with
 * row_elems > 0, new_kv [B, row_elems] bf16 into pool (device, or pinned
 * host with pool_on_host = 1); then ctx_len[b] += 1.
 * [XM-Sparse digest: each step's new KV is written back to the full
 *  history; LeanSparse Abstract: compact keys for the search.]             */
typedef struct {
    int32_t batch, max_ctx, head_dim, row_elems, keys_on_host, pool_on_host;
} ls_append_desc;

int ls_append_token(const ls_append_desc *desc, const int8_t *new_k8_dev, const void *new_kv_dev,
                    int8_t *k8, uint8_t *kc_dev, void *pool, int32_t *ctx_len_dev,
                    ls_stream_t stream);

/* Prefill indexer on device-resident keys [max_ctx, D]: for each query row
 * i (q [n_query,H,D], w [n_query,H]), the topk best keys among 0..q_pos0+i.
 * topk: out [n_query, topk], ascending, -1 padded.
 * [LeanSparse Abstract, prefill.]                                           */
int ls_prefill_index_topk(const ls_prefill_desc *desc, const int8_t *q_dev, const int8_t *w_dev,
                          const int8_t *keys_dev, int32_t *topk_dev, void *ws_dev,
                          size_t ws_bytes, ls_stream_t stream);

/* Prefill over n_layers layers with the key histories in pinned host memory
 * (keys_host[l]: [max_ctx, D] int8), streamed through the two device buffers
 * buf0 / buf1 (max_ctx*D bytes each): the copy of layer l+1 on copy_stream
 * overlaps the indexer of layer l on stream.  q[l], w[l], topk[l] as in
 * ls_prefill_index_topk.  The results equal n_layers separate calls.
 * [LeanSparse Abstract: two reusable GPU buffers, next-layer load overlapped
 * with ongoing computation.]                                               */
int ls_prefill_stream_layers(const ls_prefill_desc *desc, int32_t n_layers,
                             const int8_t *const *q_dev, const int8_t *const *w_dev,
                             const int8_t *const *keys_host, int8_t *buf0_dev, int8_t *buf1_dev,
                             int32_t *const *topk_dev, void *ws_dev, size_t ws_bytes,
                             ls_stream_t stream, ls_stream_t copy_stream);

/* ---------------------------------------------------------- measurement -- */

/* Memory-read probe: reads device memory the way the decode step does and
 * folds it into a value that decides a rare write of *sink_dev (one uint32),
 * computing nothing of the method.  rows_dev == NULL: a streaming read of
 * [base_dev, base_dev + bytes) (bytes a multiple of 16) -- the coarse pass's
 * pattern.  rows_dev != NULL: a gather of the n_rows rows rows_dev[i] of
 * row_bytes each (128 or 1152, else LS_E_UNSUPPORTED) at base_dev +
 * rows_dev[i] * row_bytes, ids clamped into the range's whole rows -- the
 * refinement's key rows and the attention's latent rows.  Timing it gives the bandwidth the hardware
 * delivers to each pattern, the context of the roofline figures.           */
int ls_read_probe(const void *base_dev, uint64_t bytes, const int32_t *rows_dev, int64_t n_rows,
                  int32_t row_bytes, uint32_t *sink_dev, ls_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LS_H */
