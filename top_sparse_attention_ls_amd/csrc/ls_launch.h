// Internal launch interface between the C-ABI host code (ls_abi.hip) and the
// kernel translation units.  Every launcher only enqueues on `st` and returns
// the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

namespace ls {

// Histogram of coarse scores: float-like monotone buckets of an int32 score,
// 6 mantissa bits, both signs (see coarse_bucket in k_index.hip).
constexpr int kCoarseBins = 3328;
// The same for int64 scores (prefill rows): 7552 buckets.
constexpr int kWideBins = 7552;
// Per-request counters sit on their own 128-byte lines (32 words apart).
constexpr int kCtrStride = 32;
// Tokens scored by one workgroup of the coarse kernel, at most (its LDS
// holds that many scores).
constexpr int kCoarseTokPerWG = 8192;
// Workgroups of the coarse kernel resident on the GPU at once: two per CU
// (two waves per SIMD) on 256 CUs.
constexpr int kCoarseSlots = 512;
// The tokens per workgroup a launch uses.
//   - kCoarseTokPerWG while that fills every slot.
//   - Else, when a row cut into floor(slots / B) pieces (rounded up to whole
//     256-token workgroup steps) keeps at least 2048 tokens per piece, those
//     pieces: all workgroups run at once with the work spread evenly, instead
//     of some CUs holding two full workgroups while others hold one.
//   - Else (little work per request) kCoarseTokPerWG halved, down to 256,
//     while the grid would hold fewer than 256 workgroups: smaller pieces
//     than that pay more in each workgroup's fixed work (its histogram, the
//     query operands) than they gain.
inline int coarse_tokens_per_wg(int B, int max_ctx) {
  const int64_t full = (int64_t)B * ((max_ctx + kCoarseTokPerWG - 1) / kCoarseTokPerWG);
  if (full >= kCoarseSlots) return kCoarseTokPerWG;
  const int pieces = (int)std::max<int64_t>(1, kCoarseSlots / std::max(B, 1));
  const int64_t per = ((int64_t)max_ctx + pieces - 1) / pieces;
  const int64_t bal = (per + 255) / 256 * 256;
  if (bal >= 2048) return (int)std::min<int64_t>(bal, kCoarseTokPerWG);
  int tpw = kCoarseTokPerWG;
  while (tpw > 256 && (int64_t)B * ((max_ctx + tpw - 1) / tpw) < 256) tpw /= 2;
  return tpw;
}
// Candidates scored by one workgroup of the refine kernel.
constexpr int kRefinePerWG = 256;
// Keys scored by one workgroup of the prefill indexer, and query rows per
// pass of it (each pass owns one score buffer of that many rows).
constexpr int kPrefillRowBlock = 512;

// Workspace of a histogram-driven selection over rows of scores of type T.
template <class T>
struct SelectWS {
  T* scores;           // [B, max_ctx]
  uint32_t* hist;      // [B, bins]             zero between calls
  uint32_t* bitmap;    // [B, bitmap_words]
  T* tie_s;            // [B, max_ctx]
  int32_t* tie_p;      // [B, max_ctx]
  uint32_t* ctr;       // [B, kCtrStride] tie count (word 0); zero between calls
  uint32_t* chunk;     // [B, n_chunks] kept count of each 16384-position chunk
  uint16_t* bucket;    // [B, max_ctx] bucket of every score (prefill rows only)
  int bitmap_words;
};
// Chunks of 16384 positions (512 bitmap words) the selection works in: one
// filter and one emit workgroup each.
constexpr int kSelectChunkWords = 512;
// ctr words of a request: tie count, beta, count above beta, emit workgroups
// done (the tie count and the last word read zero between calls)
constexpr int kCtrTies = 0, kCtrBeta = 1, kCtrAbove = 2, kCtrDone = 3;
__host__ __device__ inline int select_chunks(int bitmap_words) {
  return (bitmap_words + kSelectChunkWords - 1) / kSelectChunkWords;
}
// Chunks each emit workgroup takes: one while that is needed to fill the GPU,
// all of a row's with many rows (then no chunk counts are read).
__host__ __device__ inline int emit_chunks_per_run(int rows, int n_chunks) {
  return rows >= 256 ? n_chunks : 1;
}

using CoarseWS = SelectWS<int32_t>;  // coarse scores, kCoarseBins buckets
using WideWS = SelectWS<int64_t>;    // int64 scores, 7552 buckets

// Where the refinement reads a candidate's original int8 key row: k8
// [B, max_ctx, D] (device memory, or the device alias of pinned host
// memory), unless key_slots > 0 and the candidate's key is in the request's
// key cache kcache [B, key_slots, D] in device memory.  The cache row comes
// either from the slot table kslot [B, max_ctx] (code == nullptr) or from a
// per-candidate code [B, n_cand] written by the key-cache commit: the slot
// of a hit, -(2 + v) for a miss the refinement copies into row v, -1.
struct KeySource {
  const int8_t* k8;
  const int32_t* kslot;
  int8_t* kcache;
  int key_slots;
  const int32_t* code;
};

struct RefineWS {
  int64_t* fs;         // [B, n_cand]
  int32_t* slot;       // [B, n_cand] hot slot of each candidate (with a slot table)
  int32_t* miss_pos;   // [B, topk]
  int32_t* kcode;      // [B, n_cand] key-cache commit codes
  int32_t* miss_dst;   // [B, topk] hot-buffer slot of each inserted miss, or -1
  int32_t* src;        // [B, topk] pool position of each selected miss, -1 otherwise
};

// Cache commit (least recently used), one workgroup per request.
constexpr int kCommitDst = 0, kCommitHot = 1, kCommitKey = 2;
constexpr int kCommitMaxSlots = 16384;
constexpr int kCommitMaxEntries = 16384;
hipError_t launch_cache_commit(int mode, const int32_t* entries, int n, int32_t* pos2slot,
                               int32_t* slot2pos, uint32_t* stamp, int S, int B, int max_ctx,
                               uint32_t now, const uint32_t* now_dev, int32_t* out,
                               int32_t* rows, int32_t* n_ins, hipStream_t st);
hipError_t launch_append_token(const int8_t* new_k8, const void* new_kv, int8_t* k8,
                               uint8_t* kc, void* pool, int32_t* ctx_len, int B, int D,
                               int max_ctx, int row_elems, hipStream_t st);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

hipError_t launch_pack_coarse(const int8_t* k8, uint8_t* kc, int64_t n_rows, int dim,
                              hipStream_t st);

// With start and stop events given, the launch itself records them when the
// kernel begins and ends (the kernel's own duration, no separate commands).
hipError_t launch_coarse_scores(const int8_t* q, const int8_t* w, const uint8_t* kc,
                                const int32_t* ctx_len, const CoarseWS& ws, int B, int H,
                                int D, int max_ctx, hipStream_t st,
                                hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

hipError_t launch_topc_select(const int32_t* ctx_len, const CoarseWS& ws, int32_t* cand, int B,
                              int max_ctx, int C, hipStream_t st);

// Prefill indexer for `rows` query rows at absolute positions first_pos ..:
// score buckets, bitmap and tie lists into ws, row lengths into ctx [rows],
// top-K into topk_out [rows, K].
hipError_t launch_prefill_block(const int8_t* q, const int8_t* w, const int8_t* keys,
                                const WideWS& ws, int32_t* ctx, int32_t* topk_out, int rows,
                                int first_pos, int H, int D, int max_ctx, int K, hipStream_t st);

// The same selection over int64 scores (prefill rows).
hipError_t launch_wide_select(const int32_t* ctx_len, const WideWS& ws, int32_t* out, int B,
                              int max_ctx, int C, hipStream_t st);

// Its second kernel alone, for rows whose bitmap, tie list, chunk counts and
// counters were written by the scoring kernel itself.
hipError_t launch_wide_emit(const int32_t* ctx_len, const WideWS& ws, int32_t* out, int B,
                            int max_ctx, int C, hipStream_t st);

// Refine + top-k; with pos2slot != nullptr also the hot-buffer resolve
// (rows, n_miss, miss list in ws.miss_pos).
hipError_t launch_refine_topk(const int8_t* q, const int8_t* w, const KeySource& keys,
                              const int32_t* cand, const RefineWS& ws, int32_t* topk,
                              int64_t* topk_score, const int32_t* pos2slot, int32_t* rows,
                              int32_t* n_miss, int hot_slots, int B, int H, int D, int max_ctx,
                              int C, int K, hipStream_t st);

hipError_t launch_hot_resolve(const int32_t* topk, const int32_t* pos2slot, int32_t* rows,
                              int32_t* n_miss, int32_t* miss_pos, int hot_slots, int B,
                              int max_ctx, int K, hipStream_t st);

hipError_t launch_hot_gather(const int32_t* miss_pos, const int32_t* n_miss,
                             const int32_t* miss_dst, const void* pool, void* hot, int hot_slots,
                             int B, int max_ctx, int K, int row_elems, bool pool_on_host,
                             hipStream_t st);

// The miss gather folded into the latent attention (pool in device memory):
// src [B, K] is the pool position of each selected entry that missed the hot
// buffer (-1 for hits and padding); the entry's row in rows[] is the hot row
// the miss is copied into.  src == nullptr: no gather, the attention reads
// the hot buffer only.
struct AttnGather {
  const int32_t* src;
  const uint16_t* pool;
  int64_t pool_rows;  // rows per request in the pool (max_ctx)
};

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* rows;
  uint16_t* out;
  float* lse;
  uint16_t* part_o;   // per-split outputs, bf16
  float* part_lse;
  int B, Hq, n_kv, qk_dim, v_dim, K;
  int64_t rows_per_req, row_stride, head_stride;
  float scale;
  int n_splits;
  AttnGather gather;  // zero-initialised: no gather
};

// Rows one workgroup of the latent attention kernel handles at most; the
// split count is raised to keep every split within it.
constexpr int kAttnMaxSplitRows = 1024;

// Whether the MFMA path serves these shapes (else the generic kernel).
bool attn_uses_mfma(int Hq, int n_kv, int qk_dim, int v_dim, const void* k, const void* v);
int attn_auto_splits(int B, int Hq, int K, bool mfma);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);
hipError_t launch_combine(const AttnArgs& a, hipStream_t st);

// Memory-read probe (measurement only): a streaming read of [base, base +
// bytes) when rows == nullptr, else a gather of rows rows[0 .. n_rows) of
// row_bytes each; the data is folded into *sink.
hipError_t launch_read_probe(const void* base, uint64_t bytes, const int32_t* rows,
                             int64_t n_rows, int row_bytes, uint32_t* sink, hipStream_t st);

}  // namespace ls
