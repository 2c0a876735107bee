// Host side of the libls.so C-ABI (include/ls.h): argument validation,
// workspace planning, and the order of kernel launches for each entry point.
// Validation happens before anything is enqueued; no exception leaves here.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/ls.h"
#include "ls_launch.h"

namespace {

thread_local char g_err[512] = "";
thread_local int32_t g_hip_err = 0;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  g_hip_err = (int32_t)e;
  return fail(LS_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define LS_HIP(call, where)                          \
  do {                                               \
    hipError_t e_ = (call);                          \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------------- validation --

int check_idx(const ls_idx_desc* d) {
  if (!d) return fail(LS_E_ARG, "null indexer descriptor");
  if (d->batch < 1) return fail(LS_E_ARG, "batch must be >= 1 (got %d)", d->batch);
  if (d->max_ctx < 1 || d->max_ctx >= (1 << 28))
    return fail(LS_E_ARG, "max_ctx must be in [1, 2^28) (got %d)", d->max_ctx);
  if (d->n_cand < 1) return fail(LS_E_ARG, "n_cand must be >= 1 (got %d)", d->n_cand);
  if (d->topk < 1) return fail(LS_E_ARG, "topk must be >= 1 (got %d)", d->topk);
  if (d->n_heads < 1) return fail(LS_E_ARG, "n_heads must be >= 1 (got %d)", d->n_heads);
  if (d->n_heads > 64)
    return fail(LS_E_UNSUPPORTED, "n_heads > 64 is not supported (got %d)", d->n_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(LS_E_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->head_dim);
  if (d->keys_on_host != 0 && d->keys_on_host != 1)
    return fail(LS_E_ARG, "keys_on_host must be 0 or 1");
  if (d->key_slots < 0 || d->key_slots > (1 << 24))
    return fail(LS_E_ARG, "key_slots must be in [0, 2^24] (got %d)", d->key_slots);
  return LS_OK;
}

int check_hot(const ls_hot_desc* d) {
  if (!d) return fail(LS_E_ARG, "null hot-buffer descriptor");
  if (d->batch < 1 || d->max_ctx < 1 || d->topk < 1 || d->hot_slots < 0)
    return fail(LS_E_ARG, "bad hot-buffer shape (batch %d, max_ctx %d, topk %d, slots %d)",
                d->batch, d->max_ctx, d->topk, d->hot_slots);
  if (d->row_elems < 8 || d->row_elems % 8 != 0)
    return fail(LS_E_ARG, "row_elems must be a positive multiple of 8 (got %d)", d->row_elems);
  // the gather addresses a request's miss rows with 32-bit byte offsets
  if ((int64_t)d->topk * d->row_elems * 2 >= (int64_t)1 << 32)
    return fail(LS_E_UNSUPPORTED, "topk * row_elems * 2 bytes must stay below 2^32");
  if (d->pool_on_host != 0 && d->pool_on_host != 1)
    return fail(LS_E_ARG, "pool_on_host must be 0 or 1");
  return LS_OK;
}

int check_prefill(const ls_prefill_desc* d) {
  if (!d) return fail(LS_E_ARG, "null prefill descriptor");
  if (d->n_query < 1) return fail(LS_E_ARG, "n_query must be >= 1 (got %d)", d->n_query);
  if (d->max_ctx < 1 || d->max_ctx >= (1 << 28))
    return fail(LS_E_ARG, "max_ctx must be in [1, 2^28) (got %d)", d->max_ctx);
  if (d->q_pos0 < 0) return fail(LS_E_ARG, "q_pos0 must be >= 0 (got %d)", d->q_pos0);
  if (d->topk < 1) return fail(LS_E_ARG, "topk must be >= 1 (got %d)", d->topk);
  if (d->n_heads < 1) return fail(LS_E_ARG, "n_heads must be >= 1 (got %d)", d->n_heads);
  if (d->n_heads > 64)
    return fail(LS_E_UNSUPPORTED, "n_heads > 64 is not supported (got %d)", d->n_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(LS_E_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->head_dim);
  // the scoring kernel addresses the key history with 32-bit byte offsets
  if ((int64_t)d->max_ctx * d->head_dim >= (int64_t)1 << 31)
    return fail(LS_E_UNSUPPORTED, "max_ctx * head_dim must stay below 2^31 (got %lld)",
                (long long)d->max_ctx * d->head_dim);
  return LS_OK;
}

int check_attn(const ls_attn_desc* d) {
  if (!d) return fail(LS_E_ARG, "null attention descriptor");
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->topk < 1)
    return fail(LS_E_ARG, "bad attention shape");
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(LS_E_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", d->n_q_heads,
                d->n_kv_heads);
  if (d->qk_dim < 1 || d->v_dim < 1 || d->qk_dim > 1024 || d->v_dim > 1024)
    return fail(LS_E_UNSUPPORTED, "qk_dim and v_dim must be in [1, 1024]");
  if (d->qk_dim % 8 != 0) return fail(LS_E_ARG, "qk_dim must be a multiple of 8");
  if (d->kv_rows_per_req < 1 || d->kv_row_stride < 1 || d->kv_head_stride < 0)
    return fail(LS_E_ARG, "bad K/V strides");
  if (d->n_splits < 0) return fail(LS_E_ARG, "n_splits must be >= 0");
  if (!(d->scale == d->scale) || d->scale == __builtin_inff() || d->scale == -__builtin_inff())
    return fail(LS_E_ARG, "scale must be finite");
  return LS_OK;
}

// --------------------------------------------------------------- workspace --

struct Carve {
  size_t off = 0;
  char* base = nullptr;
  template <class T>
  T* take(size_t count) {
    off = round_up(off, 256);
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

// whole 16-byte groups per request row
int bitmap_words(int max_ctx) { return (max_ctx + 127) / 128 * 4; }

// Counters and histograms first (they must read zero between calls), bulk after.
void carve_coarse(Carve& c, const ls_idx_desc* d, ls::CoarseWS* ws) {
  const size_t B = d->batch, L = d->max_ctx;
  ls::CoarseWS w;
  w.hist = c.take<uint32_t>(B * ls::kCoarseBins);
  w.ctr = c.take<uint32_t>(B * ls::kCtrStride);
  w.scores = c.take<int32_t>(B * L);
  w.bitmap_words = bitmap_words(d->max_ctx);
  w.bitmap = c.take<uint32_t>(B * w.bitmap_words);
  w.chunk = c.take<uint32_t>(B * ls::select_chunks(w.bitmap_words));
  w.bucket = nullptr;
  w.tie_s = c.take<int32_t>(B * L);
  w.tie_p = c.take<int32_t>(B * L);
  if (ws) *ws = w;
}

// One block of prefill rows: every row is a "request" of the int64 selection.
void carve_prefill(Carve& c, const ls_prefill_desc* d, ls::WideWS* ws, int32_t** ctx) {
  const size_t R = d->n_query < ls::kPrefillRowBlock ? d->n_query : ls::kPrefillRowBlock;
  const size_t L = d->max_ctx;
  ls::WideWS w;
  w.hist = c.take<uint32_t>(R * ls::kWideBins);
  w.ctr = c.take<uint32_t>(R * ls::kCtrStride);
  w.scores = nullptr;  // the scoring kernel keeps only each score's bucket
  w.bucket = c.take<uint16_t>(R * L);
  w.bitmap_words = bitmap_words(d->max_ctx);
  w.bitmap = c.take<uint32_t>(R * w.bitmap_words);
  w.chunk = c.take<uint32_t>(R * ls::select_chunks(w.bitmap_words));
  w.tie_s = c.take<int64_t>(R * L);
  w.tie_p = c.take<int32_t>(R * L);
  int32_t* cx = c.take<int32_t>(R);
  if (ws) *ws = w;
  if (ctx) *ctx = cx;
}

void carve_refine(Carve& c, const ls_idx_desc* d, ls::RefineWS* ws) {
  const size_t B = d->batch;
  ls::RefineWS w;
  w.fs = c.take<int64_t>(B * d->n_cand);
  w.slot = c.take<int32_t>(B * d->n_cand);
  w.miss_pos = c.take<int32_t>(B * d->topk);
  w.kcode = c.take<int32_t>(B * d->n_cand);
  w.miss_dst = c.take<int32_t>(B * d->topk);
  w.src = c.take<int32_t>(B * d->topk);
  if (ws) *ws = w;
}

int attn_splits(const ls_attn_desc* d, const void* k, const void* v) {
  const bool mfma = ls::attn_uses_mfma(d->n_q_heads, d->n_kv_heads, d->qk_dim, d->v_dim, k, v);
  if (!mfma) return 1;
  int s = d->n_splits > 0 ? d->n_splits : ls::attn_auto_splits(d->batch, d->n_q_heads, d->topk, true);
  const int max_s = (d->topk + 31) / 32;
  const int min_s = (d->topk + ls::kAttnMaxSplitRows - 1) / ls::kAttnMaxSplitRows;
  if (s > max_s) s = max_s;
  return s < min_s ? min_s : s;
}

void carve_attn(Carve& c, const ls_attn_desc* d, int splits, uint16_t** part_o,
                float** part_lse) {
  const size_t BH = (size_t)d->batch * d->n_q_heads;
  const size_t s = splits > 1 ? splits : 0;
  uint16_t* po = c.take<uint16_t>(BH * s * d->v_dim);
  float* pl = c.take<float>(BH * s);
  if (part_o) *part_o = po;
  if (part_lse) *part_lse = pl;
}

// Workspace for the attention stage is sized for the auto split count of the
// MLA kernel when the caller does not fix it (the split choice does not
// depend on pointers then).
int attn_ws_splits(const ls_attn_desc* d) {
  const bool latent = d->n_kv_heads == 1 && d->qk_dim == 576 && d->v_dim == 512 &&
                      d->n_q_heads % 16 == 0;
  if (!latent) return 1;
  int s = d->n_splits > 0 ? d->n_splits : ls::attn_auto_splits(d->batch, d->n_q_heads, d->topk, true);
  const int max_s = (d->topk + 31) / 32;
  const int min_s = (d->topk + ls::kAttnMaxSplitRows - 1) / ls::kAttnMaxSplitRows;
  if (s > max_s) s = max_s;
  return s < min_s ? min_s : s;
}

size_t ws_size(int32_t op, const void* desc) {
  Carve c;
  switch (op) {
    case LS_OP_COARSE: {
      const ls_idx_desc* d = (const ls_idx_desc*)desc;
      if (check_idx(d)) return 0;
      carve_coarse(c, d, nullptr);
      break;
    }
    case LS_OP_REFINE: {
      const ls_idx_desc* d = (const ls_idx_desc*)desc;
      if (check_idx(d)) return 0;
      carve_refine(c, d, nullptr);
      break;
    }
    case LS_OP_HOT: {
      const ls_hot_desc* d = (const ls_hot_desc*)desc;
      if (check_hot(d)) return 0;
      c.take<int32_t>((size_t)d->batch * d->topk);
      break;
    }
    case LS_OP_ATTN: {
      const ls_attn_desc* d = (const ls_attn_desc*)desc;
      if (check_attn(d)) return 0;
      carve_attn(c, d, attn_ws_splits(d), nullptr, nullptr);
      break;
    }
    case LS_OP_STEP: {
      const ls_step_desc* d = (const ls_step_desc*)desc;
      if (!d) {
        fail(LS_E_ARG, "null step descriptor");
        return 0;
      }
      if (check_idx(&d->idx) || check_attn(&d->attn)) return 0;
      if (d->use_hot && check_hot(&d->hot)) return 0;
      carve_coarse(c, &d->idx, nullptr);
      carve_refine(c, &d->idx, nullptr);
      carve_attn(c, &d->attn, attn_ws_splits(&d->attn), nullptr, nullptr);
      break;
    }
    case LS_OP_PREFILL: {
      const ls_prefill_desc* d = (const ls_prefill_desc*)desc;
      if (check_prefill(d)) return 0;
      carve_prefill(c, d, nullptr, nullptr);
      break;
    }
    default:
      fail(LS_E_ARG, "unknown operation id %d", op);
      return 0;
  }
  // never 0 for a valid descriptor: 0 is the error value
  return c.off < 256 ? 256 : round_up(c.off, 256);
}

int check_ws(int32_t op, const void* desc, void* ws, size_t ws_bytes) {
  size_t need = ws_size(op, desc);
  if (need == 0) return LS_E_ARG;
  if (!ws) return fail(LS_E_WORKSPACE, "null workspace (%zu bytes needed)", need);
  if (!aligned16(ws)) return fail(LS_E_ARG, "workspace must be 16-byte aligned");
  if (ws_bytes < need)
    return fail(LS_E_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", ws_bytes, need);
  return LS_OK;
}

#define LS_TRY(x)            \
  do {                       \
    int r_ = (x);            \
    if (r_ != LS_OK) return r_; \
  } while (0)

#define LS_NONNULL(p)                                                  \
  do {                                                                 \
    if (!(p)) return fail(LS_E_ARG, "null pointer argument: %s", #p);  \
  } while (0)

#define LS_ALIGNED(p)                                                            \
  do {                                                                           \
    if (!aligned16(p)) return fail(LS_E_ARG, "%s must be 16-byte aligned", #p);  \
  } while (0)

// -------------------------------------------------------- stage launchers --

int run_coarse(const ls_idx_desc* d, const int8_t* q, const int8_t* w, const uint8_t* kc,
               const int32_t* ctx_len, int32_t* cand, const ls::CoarseWS& ws, hipStream_t st,
               ls_event_t* ev) {
  // events [0] and [1] together: the launch records them at the coarse
  // kernel's own start and end; either alone: a record command in the stream
  const bool both = ev && ev[0] && ev[1];
  if (ev && ev[0] && !both) LS_HIP(hipEventRecord((hipEvent_t)ev[0], st), "event record");
  LS_HIP(ls::launch_coarse_scores(q, w, kc, ctx_len, ws, d->batch, d->n_heads, d->head_dim,
                                  d->max_ctx, st, both ? (hipEvent_t)ev[0] : nullptr,
                                  both ? (hipEvent_t)ev[1] : nullptr),
         "coarse score launch");
  if (ev && ev[1] && !both) LS_HIP(hipEventRecord((hipEvent_t)ev[1], st), "event record");
  LS_HIP(ls::launch_topc_select(ctx_len, ws, cand, d->batch, d->max_ctx, d->n_cand, st),
         "candidate select launch");
  return LS_OK;
}

int check_idx_ptrs(const int8_t* q, const int8_t* w, const int32_t* ctx_len) {
  LS_NONNULL(q);
  LS_NONNULL(w);
  LS_NONNULL(ctx_len);
  LS_ALIGNED(q);
  return LS_OK;
}

// A buffer declared host-resident (the pool, the original int8 keys) must
// be pinned, device-mapped host memory; the kernels read it through its
// device alias.  Anything else is rejected here, before a kernel could touch
// an unmapped address.
int resolve_host(const void* p, int on_host, const void** dev_ptr, const char* what) {
  if (!on_host) {
    *dev_ptr = p;
    return LS_OK;
  }
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(LS_E_ARG, "%s is declared host-resident but is not pinned host memory (%s)", what,
                hipGetErrorString(e));
  }
  if (attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr)
    return fail(LS_E_ARG, "%s is declared host-resident but is not device-mapped pinned host memory",
                what);
  // a pointer inside a pinned allocation (a slice of a larger tensor): the
  // alias keeps its offset from the host address the attributes report
  const char* dev = (const char*)attr.devicePointer;
  if (attr.hostPointer) dev += (const char*)p - (const char*)attr.hostPointer;
  *dev_ptr = dev;
  return LS_OK;
}

int resolve_pool(const void* pool, int on_host, const void** dev_ptr) {
  return resolve_host(pool, on_host, dev_ptr, "the pool (pool_on_host = 1)");
}

// The refinement's key source: k8 (through its device alias when it is host
// memory) and, with key_slots > 0, the device-resident key cache.
int resolve_keys(const ls_idx_desc* d, const int8_t* k8, const int32_t* kpos2slot,
                 const int8_t* kcache, ls::KeySource* ks) {
  ks->code = nullptr;
  LS_NONNULL(k8);
  LS_ALIGNED(k8);
  const void* p = nullptr;
  LS_TRY(resolve_host(k8, d->keys_on_host, &p, "k8 (keys_on_host = 1)"));
  ks->k8 = (const int8_t*)p;
  ks->key_slots = d->key_slots;
  ks->kslot = nullptr;
  ks->kcache = nullptr;
  if (d->key_slots > 0) {
    LS_NONNULL(kpos2slot);
    LS_NONNULL(kcache);
    LS_ALIGNED(kpos2slot);
    LS_ALIGNED(kcache);
    ks->kslot = kpos2slot;
    ks->kcache = (int8_t*)kcache;
  }
  return LS_OK;
}

}  // namespace

extern "C" {

int32_t ls_abi_version(void) { return LS_ABI_VERSION; }
const char* ls_last_error(void) { return g_err; }
int32_t ls_last_hip_error(void) { return g_hip_err; }

size_t ls_workspace_size(int32_t op, const void* desc) {
  try {
    return ws_size(op, desc);
  } catch (...) {
    fail(LS_E_ARG, "internal error");
    return 0;
  }
}

int ls_workspace_init(void* ws_dev, size_t ws_bytes, ls_stream_t stream) {
  if (!ws_dev) return fail(LS_E_ARG, "null workspace");
  if (!aligned16(ws_dev)) return fail(LS_E_ARG, "workspace must be 16-byte aligned");
  if (ws_bytes == 0) return LS_OK;
  LS_HIP(ls::launch_fill_zero(ws_dev, ws_bytes, (hipStream_t)stream), "workspace clear");
  return LS_OK;
}

int ls_pack_coarse(const int8_t* k8_dev, uint8_t* kc_dev, int64_t n_rows, int32_t dim,
                   ls_stream_t stream) {
  LS_NONNULL(k8_dev);
  LS_NONNULL(kc_dev);
  if (n_rows < 0) return fail(LS_E_ARG, "n_rows must be >= 0");
  if (dim < 4 || dim % 4 != 0) return fail(LS_E_ARG, "dim must be a positive multiple of 4");
  if (((uintptr_t)k8_dev & 3u) || ((uintptr_t)kc_dev & 1u))
    return fail(LS_E_ARG, "k8 must be 4-byte and kc 2-byte aligned");
  if (n_rows == 0) return LS_OK;
  LS_HIP(ls::launch_pack_coarse(k8_dev, kc_dev, n_rows, dim, (hipStream_t)stream), "pack launch");
  return LS_OK;
}

int ls_index_coarse(const ls_idx_desc* desc, const int8_t* q_dev, const int8_t* w_dev,
                    const uint8_t* kc_dev, const int32_t* ctx_len_dev, int32_t* cand_dev,
                    void* ws_dev, size_t ws_bytes, ls_stream_t stream) {
  LS_TRY(check_idx(desc));
  LS_TRY(check_idx_ptrs(q_dev, w_dev, ctx_len_dev));
  LS_NONNULL(kc_dev);
  LS_NONNULL(cand_dev);
  LS_ALIGNED(kc_dev);
  LS_TRY(check_ws(LS_OP_COARSE, desc, ws_dev, ws_bytes));
  Carve c;
  c.base = (char*)ws_dev;
  ls::CoarseWS ws;
  carve_coarse(c, desc, &ws);
  return run_coarse(desc, q_dev, w_dev, kc_dev, ctx_len_dev, cand_dev, ws, (hipStream_t)stream,
                    nullptr);
}

int ls_refine_topk(const ls_idx_desc* desc, const int8_t* q_dev, const int8_t* w_dev,
                   const int8_t* k8_dev, const int32_t* kpos2slot_dev, const int8_t* kcache_dev,
                   const int32_t* cand_dev, const int32_t* ctx_len_dev, int32_t* topk_dev,
                   int64_t* topk_score_dev, void* ws_dev, size_t ws_bytes, ls_stream_t stream) {
  LS_TRY(check_idx(desc));
  LS_TRY(check_idx_ptrs(q_dev, w_dev, ctx_len_dev));
  LS_NONNULL(cand_dev);
  LS_NONNULL(topk_dev);
  LS_TRY(check_ws(LS_OP_REFINE, desc, ws_dev, ws_bytes));
  ls::KeySource k8;
  LS_TRY(resolve_keys(desc, k8_dev, kpos2slot_dev, kcache_dev, &k8));
  Carve c;
  c.base = (char*)ws_dev;
  ls::RefineWS ws;
  carve_refine(c, desc, &ws);
  LS_HIP(ls::launch_refine_topk(q_dev, w_dev, k8, cand_dev, ws, topk_dev, topk_score_dev,
                                nullptr, nullptr, nullptr, 0, desc->batch, desc->n_heads,
                                desc->head_dim, desc->max_ctx, desc->n_cand, desc->topk,
                                (hipStream_t)stream),
         "refine launch");
  return LS_OK;
}

int ls_hot_gather(const ls_hot_desc* desc, const int32_t* topk_dev, const int32_t* pos2slot_dev,
                  void* hot_kv_dev, const void* pool_kv_dev, int32_t* rows_dev,
                  int32_t* n_miss_dev, void* ws_dev, size_t ws_bytes, ls_stream_t stream) {
  LS_TRY(check_hot(desc));
  LS_NONNULL(topk_dev);
  LS_NONNULL(pos2slot_dev);
  LS_NONNULL(hot_kv_dev);
  LS_NONNULL(pool_kv_dev);
  LS_NONNULL(rows_dev);
  LS_NONNULL(n_miss_dev);
  LS_ALIGNED(hot_kv_dev);
  LS_ALIGNED(pool_kv_dev);
  LS_TRY(check_ws(LS_OP_HOT, desc, ws_dev, ws_bytes));
  const void* pool = nullptr;
  LS_TRY(resolve_pool(pool_kv_dev, desc->pool_on_host, &pool));
  Carve c;
  c.base = (char*)ws_dev;
  int32_t* miss_pos = c.take<int32_t>((size_t)desc->batch * desc->topk);
  hipStream_t st = (hipStream_t)stream;
  LS_HIP(ls::launch_hot_resolve(topk_dev, pos2slot_dev, rows_dev, n_miss_dev, miss_pos,
                                desc->hot_slots, desc->batch, desc->max_ctx, desc->topk, st),
         "hot resolve launch");
  LS_HIP(ls::launch_hot_gather(miss_pos, n_miss_dev, nullptr, pool, hot_kv_dev, desc->hot_slots,
                               desc->batch, desc->max_ctx, desc->topk, desc->row_elems,
                               desc->pool_on_host != 0, st),
         "miss gather launch");
  return LS_OK;
}

static int check_commit_shape(int32_t n_slots, int32_t n, uint32_t now, const char* what) {
  if (n_slots < 1 || n_slots > ls::kCommitMaxSlots)
    return fail(LS_E_ARG, "%s: a committed cache needs 1..%d slots (got %d)", what,
                ls::kCommitMaxSlots, n_slots);
  if (n < 1 || n > ls::kCommitMaxEntries)
    return fail(LS_E_ARG, "%s: a commit takes 1..%d entries per request (got %d)", what,
                ls::kCommitMaxEntries, n);
  if (now == 0xFFFFFFFFu) return fail(LS_E_ARG, "%s: now must be below 2^32 - 1", what);
  return LS_OK;
}

int ls_cache_commit(int32_t batch, int32_t max_ctx, int32_t n_slots, int32_t n, uint32_t now,
                    const int32_t* entries_dev, int32_t* pos2slot_dev, int32_t* slot2pos_dev,
                    uint32_t* stamp_dev, int32_t* dst_dev, int32_t* n_inserted_dev,
                    ls_stream_t stream) {
  if (batch < 1 || max_ctx < 1)
    return fail(LS_E_ARG, "bad commit shape (batch %d, max_ctx %d)", batch, max_ctx);
  LS_TRY(check_commit_shape(n_slots, n, now, "cache commit"));
  LS_NONNULL(entries_dev);
  LS_NONNULL(pos2slot_dev);
  LS_NONNULL(slot2pos_dev);
  LS_NONNULL(stamp_dev);
  LS_NONNULL(dst_dev);
  LS_HIP(ls::launch_cache_commit(ls::kCommitDst, entries_dev, n, pos2slot_dev, slot2pos_dev,
                                 stamp_dev, n_slots, batch, max_ctx, now, nullptr, dst_dev,
                                 nullptr,
                                 n_inserted_dev, (hipStream_t)stream),
         "cache commit launch");
  return LS_OK;
}

int ls_append_token(const ls_append_desc* desc, const int8_t* new_k8_dev, const void* new_kv_dev,
                    int8_t* k8, uint8_t* kc_dev, void* pool, int32_t* ctx_len_dev,
                    ls_stream_t stream) {
  if (!desc) return fail(LS_E_ARG, "null append descriptor");
  if (desc->batch < 1 || desc->max_ctx < 1)
    return fail(LS_E_ARG, "bad append shape (batch %d, max_ctx %d)", desc->batch, desc->max_ctx);
  if (desc->head_dim != 64 && desc->head_dim != 128)
    return fail(LS_E_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", desc->head_dim);
  if (desc->row_elems < 0 || desc->row_elems % 8 != 0)
    return fail(LS_E_ARG, "row_elems must be 0 or a positive multiple of 8 (got %d)",
                desc->row_elems);
  if ((desc->keys_on_host != 0 && desc->keys_on_host != 1) ||
      (desc->pool_on_host != 0 && desc->pool_on_host != 1))
    return fail(LS_E_ARG, "keys_on_host and pool_on_host must be 0 or 1");
  LS_NONNULL(new_k8_dev);
  LS_NONNULL(k8);
  LS_NONNULL(kc_dev);
  LS_NONNULL(ctx_len_dev);
  LS_ALIGNED(new_k8_dev);
  LS_ALIGNED(k8);
  LS_ALIGNED(kc_dev);
  const void* k8d = nullptr;
  LS_TRY(resolve_host(k8, desc->keys_on_host, &k8d, "k8 (keys_on_host = 1)"));
  const void* pd = nullptr;
  if (desc->row_elems > 0) {
    LS_NONNULL(new_kv_dev);
    LS_NONNULL(pool);
    LS_ALIGNED(new_kv_dev);
    LS_ALIGNED(pool);
    LS_TRY(resolve_pool(pool, desc->pool_on_host, &pd));
  }
  LS_HIP(ls::launch_append_token(new_k8_dev, new_kv_dev, (int8_t*)k8d, kc_dev, (void*)pd,
                                 ctx_len_dev, desc->batch, desc->head_dim, desc->max_ctx,
                                 desc->row_elems, (hipStream_t)stream),
         "append launch");
  return LS_OK;
}

static int attn_args(const ls_attn_desc* d, const void* q, const void* k, const void* v,
                     const int32_t* rows, void* out, float* lse, void* ws, ls::AttnArgs* a) {
  a->q = (const uint16_t*)q;
  a->k = (const uint16_t*)k;
  a->v = (const uint16_t*)v;
  a->rows = rows;
  a->out = (uint16_t*)out;
  a->lse = lse;
  a->B = d->batch;
  a->Hq = d->n_q_heads;
  a->n_kv = d->n_kv_heads;
  a->qk_dim = d->qk_dim;
  a->v_dim = d->v_dim;
  a->K = d->topk;
  a->rows_per_req = d->kv_rows_per_req;
  a->row_stride = d->kv_row_stride;
  a->head_stride = d->kv_head_stride;
  a->scale = d->scale;
  const bool mfma = ls::attn_uses_mfma(d->n_q_heads, d->n_kv_heads, d->qk_dim, d->v_dim, k, v);
  if (!mfma && d->topk > 8192)
    return fail(LS_E_UNSUPPORTED, "topk > 8192 needs the latent (576/512, one kv head) layout");
  if (!mfma && (d->v_dim % 8 != 0 || d->kv_row_stride % 8 != 0 || d->kv_head_stride % 8 != 0))
    return fail(LS_E_UNSUPPORTED, "the generic attention reads 16-byte pieces: v_dim and the "
                                  "row and head strides must be multiples of 8");
  a->n_splits = attn_splits(d, k, v);
  a->gather = ls::AttnGather{};  // no gather unless the step folds it in
  (void)ws;
  return LS_OK;
}

static int run_attention(const ls::AttnArgs& a, hipStream_t st, ls_event_t* ev) {
  LS_HIP(ls::launch_attention(a, st), "attention launch");
  if (ev && ev[5]) LS_HIP(hipEventRecord((hipEvent_t)ev[5], st), "event record");
  if (a.n_splits > 1) LS_HIP(ls::launch_combine(a, st), "combine launch");
  return LS_OK;
}

int ls_sparse_attn_decode(const ls_attn_desc* desc, const void* q_dev, const void* k_base_dev,
                          const void* v_base_dev, const int32_t* rows_dev, void* out_dev,
                          float* lse_dev, void* ws_dev, size_t ws_bytes, ls_stream_t stream) {
  LS_TRY(check_attn(desc));
  LS_NONNULL(q_dev);
  LS_NONNULL(k_base_dev);
  LS_NONNULL(v_base_dev);
  LS_NONNULL(rows_dev);
  LS_NONNULL(out_dev);
  LS_NONNULL(lse_dev);
  LS_ALIGNED(q_dev);
  LS_ALIGNED(k_base_dev);
  LS_ALIGNED(v_base_dev);
  LS_ALIGNED(out_dev);
  LS_TRY(check_ws(LS_OP_ATTN, desc, ws_dev, ws_bytes));
  ls::AttnArgs a;
  LS_TRY(attn_args(desc, q_dev, k_base_dev, v_base_dev, rows_dev, out_dev, lse_dev, ws_dev, &a));
  if (a.n_splits > attn_ws_splits(desc))
    return fail(LS_E_WORKSPACE, "split count exceeds the workspace plan");
  Carve c;
  c.base = (char*)ws_dev;
  carve_attn(c, desc, attn_ws_splits(desc), &a.part_o, &a.part_lse);
  return run_attention(a, (hipStream_t)stream, nullptr);
}

}  // extern "C"

namespace {

// The whole step on workspace ws_dev.  clear_bytes > 0: a fill kernel first
// zeroes ws_dev[0, clear_bytes) -- after every check, so that a rejected call
// enqueues nothing.
int decode_step_impl(const ls_step_desc* desc, const ls_step_io* io, void* ws_dev,
                     size_t ws_bytes, ls_stream_t stream, size_t clear_bytes) {
  if (!desc) return fail(LS_E_ARG, "null step descriptor");
  if (!io) return fail(LS_E_ARG, "null step io");
  const ls_idx_desc* id = &desc->idx;
  const ls_attn_desc* ad = &desc->attn;
  LS_TRY(check_idx(id));
  LS_TRY(check_attn(ad));
  if (desc->use_hot != 0 && desc->use_hot != 1) return fail(LS_E_ARG, "use_hot must be 0 or 1");
  if (ad->batch != id->batch || ad->topk != id->topk)
    return fail(LS_E_ARG, "attention batch/topk must match the indexer's");
  LS_TRY(check_idx_ptrs(io->q_idx_dev, io->w_idx_dev, io->ctx_len_dev));
  LS_NONNULL(io->kc_dev);
  LS_NONNULL(io->cand_dev);
  LS_NONNULL(io->topk_dev);
  LS_NONNULL(io->q_attn_dev);
  LS_NONNULL(io->out_dev);
  LS_NONNULL(io->lse_dev);
  LS_ALIGNED(io->kc_dev);
  LS_ALIGNED(io->q_attn_dev);
  LS_ALIGNED(io->out_dev);
  const void *kb, *vb;
  if (desc->use_hot) {
    const ls_hot_desc* hd = &desc->hot;
    LS_TRY(check_hot(hd));
    if (hd->batch != id->batch || hd->topk != id->topk || hd->max_ctx != id->max_ctx)
      return fail(LS_E_ARG, "hot-buffer batch/topk/max_ctx must match the indexer's");
    if (hd->row_elems != ad->qk_dim || ad->kv_row_stride != hd->row_elems ||
        ad->kv_rows_per_req != (int64_t)hd->hot_slots + hd->topk || ad->n_kv_heads != 1)
      return fail(LS_E_ARG, "with a hot buffer, attention must read its latent rows "
                            "(one kv head, row stride = row_elems, hot_slots + topk rows)");
    LS_NONNULL(io->pos2slot_dev);
    LS_NONNULL(io->hot_kv_dev);
    LS_NONNULL(io->pool_kv_dev);
    LS_NONNULL(io->rows_dev);
    LS_NONNULL(io->n_miss_dev);
    LS_ALIGNED(io->hot_kv_dev);
    LS_ALIGNED(io->pool_kv_dev);
    kb = vb = io->hot_kv_dev;
  } else {
    LS_NONNULL(io->k_cache_dev);
    LS_NONNULL(io->v_cache_dev);
    LS_ALIGNED(io->k_cache_dev);
    LS_ALIGNED(io->v_cache_dev);
    if (ad->kv_rows_per_req != id->max_ctx)
      return fail(LS_E_ARG, "without a hot buffer, kv_rows_per_req must equal max_ctx");
    kb = io->k_cache_dev;
    vb = io->v_cache_dev;
  }
  const ls_commit_desc* cm = &desc->commit;
  if ((cm->hot != 0 && cm->hot != 1) || (cm->keys != 0 && cm->keys != 1))
    return fail(LS_E_ARG, "commit.hot and commit.keys must be 0 or 1");
  if (cm->hot) {
    if (!desc->use_hot) return fail(LS_E_ARG, "commit.hot needs the hot buffer (use_hot = 1)");
    LS_TRY(check_commit_shape(desc->hot.hot_slots, id->topk, cm->now, "commit.hot"));
    if ((int64_t)(desc->hot.hot_slots + id->topk) * desc->hot.row_elems * 2 >= ((int64_t)1 << 32))
      return fail(LS_E_ARG, "commit.hot: the hot buffer of a request must stay below 4 GiB");
    LS_NONNULL(io->slot2pos_dev);
    LS_NONNULL(io->stamp_dev);
  }
  if (cm->keys) {
    if (id->key_slots < 1) return fail(LS_E_ARG, "commit.keys needs a key cache (key_slots > 0)");
    LS_TRY(check_commit_shape(id->key_slots, id->n_cand, cm->now, "commit.keys"));
    LS_NONNULL(io->kslot2pos_dev);
    LS_NONNULL(io->kstamp_dev);
  }
  LS_TRY(check_ws(LS_OP_STEP, desc, ws_dev, ws_bytes));
  const void* pool = nullptr;
  if (desc->use_hot) LS_TRY(resolve_pool(io->pool_kv_dev, desc->hot.pool_on_host, &pool));
  ls::KeySource k8;
  LS_TRY(resolve_keys(id, io->k8_dev, io->kpos2slot_dev, io->kcache_dev, &k8));

  Carve c;
  c.base = (char*)ws_dev;
  ls::CoarseWS cws;
  ls::RefineWS rws;
  carve_coarse(c, id, &cws);
  carve_refine(c, id, &rws);
  ls::AttnArgs a;
  const int32_t* rows = desc->use_hot ? io->rows_dev : io->topk_dev;
  LS_TRY(attn_args(ad, io->q_attn_dev, kb, vb, rows, io->out_dev, io->lse_dev, ws_dev, &a));
  if (a.n_splits > attn_ws_splits(ad))
    return fail(LS_E_WORKSPACE, "split count exceeds the workspace plan");
  carve_attn(c, ad, attn_ws_splits(ad), &a.part_o, &a.part_lse);

  hipStream_t st = (hipStream_t)stream;
  ls_event_t* ev = io->stage_events;
  if (clear_bytes) LS_HIP(ls::launch_fill_zero(ws_dev, clear_bytes, st), "scratch clear");
  LS_TRY(run_coarse(id, io->q_idx_dev, io->w_idx_dev, io->kc_dev, io->ctx_len_dev, io->cand_dev,
                    cws, st, ev));
  if (ev && ev[2]) LS_HIP(hipEventRecord((hipEvent_t)ev[2], st), "event record");
  if (cm->keys) {
    // the candidates' key-cache hits and the rows their misses move into;
    // the refinement reads by these codes and fills the rows
    LS_HIP(ls::launch_cache_commit(ls::kCommitKey, io->cand_dev, id->n_cand, io->kpos2slot_dev,
                                   io->kslot2pos_dev, io->kstamp_dev, id->key_slots, id->batch,
                                   id->max_ctx, cm->now, io->now_dev, rws.kcode, nullptr,
                                   io->n_key_miss_dev,
                                   st),
           "key-cache commit launch");
    k8.code = rws.kcode;
  }
  LS_HIP(ls::launch_refine_topk(io->q_idx_dev, io->w_idx_dev, k8, io->cand_dev, rws,
                                io->topk_dev, io->topk_score_dev,
                                desc->use_hot ? io->pos2slot_dev : nullptr,
                                desc->use_hot ? io->rows_dev : nullptr,
                                desc->use_hot ? io->n_miss_dev : nullptr, desc->hot.hot_slots,
                                id->batch, id->n_heads, id->head_dim, id->max_ctx, id->n_cand,
                                id->topk, st),
         "refine launch");
  if (ev && ev[3]) LS_HIP(hipEventRecord((hipEvent_t)ev[3], st), "event record");
  if (cm->hot)
    // the misses' victim slots (rows[] rewritten to them), before the gather
    // writes the rows there
    LS_HIP(ls::launch_cache_commit(ls::kCommitHot, io->topk_dev, id->topk, io->pos2slot_dev,
                                   io->slot2pos_dev, io->stamp_dev, desc->hot.hot_slots,
                                   id->batch, id->max_ctx, cm->now, io->now_dev, rws.miss_dst,
                                   io->rows_dev,
                                   nullptr, st),
           "hot-buffer commit launch");
  // With the pool in device memory the attention itself reads the misses
  // from the pool and copies them into their hot-buffer rows (one launch
  // fewer); a pool in host memory keeps the separate gather, so that the
  // attention never waits on PCIe.
  const bool fuse_gather = desc->use_hot && !desc->hot.pool_on_host &&
                           ls::attn_uses_mfma(ad->n_q_heads, ad->n_kv_heads, ad->qk_dim,
                                              ad->v_dim, io->hot_kv_dev, io->hot_kv_dev) &&
                           ad->n_q_heads <= 128 &&
                           (int64_t)id->max_ctx * desc->hot.row_elems * 2 < ((int64_t)1 << 32) &&
                           (int64_t)(desc->hot.hot_slots + id->topk) * desc->hot.row_elems * 2 <
                               ((int64_t)1 << 32);
  if (fuse_gather) {
    a.gather.src = rws.src;
    a.gather.pool = (const uint16_t*)pool;
    a.gather.pool_rows = id->max_ctx;
  } else if (desc->use_hot) {
    LS_HIP(ls::launch_hot_gather(rws.miss_pos, io->n_miss_dev, cm->hot ? rws.miss_dst : nullptr,
                                 pool, io->hot_kv_dev, desc->hot.hot_slots, id->batch,
                                 id->max_ctx, id->topk, desc->hot.row_elems,
                                 desc->hot.pool_on_host != 0, st),
           "miss gather launch");
  }
  if (ev && ev[4]) LS_HIP(hipEventRecord((hipEvent_t)ev[4], st), "event record");
  LS_TRY(run_attention(a, st, ev));
  if (ev && ev[6]) LS_HIP(hipEventRecord((hipEvent_t)ev[6], st), "event record");
  return LS_OK;
}

// Bytes at the start of a step workspace that must read zero when a call
// begins (the score histograms and the counters, carved first).
size_t step_zero_prefix(const ls_step_desc* d) {
  Carve c;
  c.take<uint32_t>((size_t)d->idx.batch * ls::kCoarseBins);
  c.take<uint32_t>((size_t)d->idx.batch * ls::kCtrStride);
  return round_up(c.off, 256);
}

// Static scratch of the allocation-free step (see ls_decode_step_noalloc):
// one copy per device, held until the process ends.  The array's name is a
// host-side stand-in; kernels get the device address from
// hipGetSymbolAddress, looked up once per device.
constexpr size_t kStaticScratchBytes = (size_t)128 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = -1;
  LS_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LS_E_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    LS_HIP(hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)), "scratch symbol address");
    if (!ptr) return fail(LS_E_HIP, "scratch symbol address is null");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return LS_OK;
}

}  // namespace

extern "C" {

int ls_decode_step(const ls_step_desc* desc, const ls_step_io* io, void* ws_dev,
                   size_t ws_bytes, ls_stream_t stream) {
  try {
    return decode_step_impl(desc, io, ws_dev, ws_bytes, stream, 0);
  } catch (...) {
    return fail(LS_E_ARG, "internal error");
  }
}

int ls_decode_step_noalloc(const ls_step_desc* desc, const ls_step_io* io, ls_stream_t stream) {
  try {
    if (!desc) return fail(LS_E_ARG, "null step descriptor");
    const size_t need = ws_size(LS_OP_STEP, desc);
    if (need == 0) return LS_E_ARG;
    if (need > kStaticScratchBytes)
      return fail(LS_E_UNSUPPORTED,
                  "the step needs %zu bytes of scratch, more than the %zu bytes of the static "
                  "scratch of ls_decode_step_noalloc", need, kStaticScratchBytes);
    void* ws = nullptr;
    LS_TRY(static_scratch(&ws));
    return decode_step_impl(desc, io, ws, kStaticScratchBytes, stream, step_zero_prefix(desc));
  } catch (...) {
    return fail(LS_E_ARG, "internal error");
  }
}

int ls_read_probe(const void* base_dev, uint64_t bytes, const int32_t* rows_dev, int64_t n_rows,
                  int32_t row_bytes, uint32_t* sink_dev, ls_stream_t stream) {
  LS_NONNULL(base_dev);
  LS_NONNULL(sink_dev);
  LS_ALIGNED(base_dev);
  if (bytes % 16 != 0) return fail(LS_E_ARG, "bytes must be a multiple of 16");
  if (rows_dev) {
    if (row_bytes < 16 || row_bytes % 16 != 0)
      return fail(LS_E_ARG, "row_bytes must be a positive multiple of 16 (got %d)", row_bytes);
    if (n_rows < 0) return fail(LS_E_ARG, "n_rows must be >= 0");
    if ((uint64_t)row_bytes > bytes) return fail(LS_E_ARG, "the range holds no whole row");
    if (row_bytes != 128 && row_bytes != 1152)
      return fail(LS_E_UNSUPPORTED, "row_bytes must be 128 or 1152 (the step's row sizes)");
    if ((uint64_t)n_rows * (row_bytes / 16) >= ((uint64_t)1 << 31) ||
        bytes / (uint64_t)row_bytes >= ((uint64_t)1 << 31))
      return fail(LS_E_UNSUPPORTED, "too many rows for the probe");
  }
  LS_HIP(ls::launch_read_probe(base_dev, bytes, rows_dev, n_rows, row_bytes, sink_dev,
                               (hipStream_t)stream),
         "read probe launch");
  return LS_OK;
}

int ls_prefill_index_topk(const ls_prefill_desc* desc, const int8_t* q_dev, const int8_t* w_dev,
                          const int8_t* keys_dev, int32_t* topk_dev, void* ws_dev,
                          size_t ws_bytes, ls_stream_t stream) {
  LS_TRY(check_prefill(desc));
  LS_NONNULL(q_dev);
  LS_NONNULL(w_dev);
  LS_NONNULL(keys_dev);
  LS_NONNULL(topk_dev);
  LS_ALIGNED(q_dev);
  LS_ALIGNED(keys_dev);
  LS_TRY(check_ws(LS_OP_PREFILL, desc, ws_dev, ws_bytes));
  Carve c;
  c.base = (char*)ws_dev;
  ls::WideWS ws;
  int32_t* ctx = nullptr;
  carve_prefill(c, desc, &ws, &ctx);
  const int H = desc->n_heads, D = desc->head_dim, K = desc->topk;
  for (int r0 = 0; r0 < desc->n_query; r0 += ls::kPrefillRowBlock) {
    const int rows = std::min(ls::kPrefillRowBlock, desc->n_query - r0);
    LS_HIP(ls::launch_prefill_block(q_dev + (size_t)r0 * H * D, w_dev + (size_t)r0 * H, keys_dev,
                                    ws, ctx, topk_dev + (size_t)r0 * K, rows, desc->q_pos0 + r0,
                                    H, D, desc->max_ctx, K, (hipStream_t)stream),
           "prefill launch");
  }
  return LS_OK;
}

int ls_prefill_stream_layers(const ls_prefill_desc* desc, int32_t n_layers,
                             const int8_t* const* q_dev, const int8_t* const* w_dev,
                             const int8_t* const* keys_host, int8_t* buf0_dev, int8_t* buf1_dev,
                             int32_t* const* topk_dev, void* ws_dev, size_t ws_bytes,
                             ls_stream_t stream, ls_stream_t copy_stream) {
  LS_TRY(check_prefill(desc));
  if (n_layers < 1) return fail(LS_E_ARG, "n_layers must be >= 1 (got %d)", n_layers);
  LS_NONNULL(q_dev);
  LS_NONNULL(w_dev);
  LS_NONNULL(keys_host);
  LS_NONNULL(topk_dev);
  LS_NONNULL(buf0_dev);
  LS_NONNULL(buf1_dev);
  LS_ALIGNED(buf0_dev);
  LS_ALIGNED(buf1_dev);
  if (stream == copy_stream)
    return fail(LS_E_ARG, "the copy stream must differ from the compute stream");
  for (int l = 0; l < n_layers; l++) {
    if (!q_dev[l] || !w_dev[l] || !keys_host[l] || !topk_dev[l])
      return fail(LS_E_ARG, "null pointer for layer %d", l);
  }
  LS_TRY(check_ws(LS_OP_PREFILL, desc, ws_dev, ws_bytes));
  hipStream_t st = (hipStream_t)stream, cp = (hipStream_t)copy_stream;
  const size_t bytes = (size_t)desc->max_ctx * desc->head_dim;
  // copied[l]: layer l's keys are in its buffer; done[l]: layer l no longer
  // reads its buffer, so layer l + 2 may overwrite it
  std::vector<hipEvent_t> copied, done;
  try {
    copied.assign(n_layers, nullptr);
    done.assign(n_layers, nullptr);
  } catch (const std::bad_alloc&) {
    return fail(LS_E_ARG, "cannot track %d layers", n_layers);
  }
  int rc = LS_OK;
  for (int l = 0; l < n_layers && rc == LS_OK; l++) {
    int8_t* buf = (l & 1) ? buf1_dev : buf0_dev;
    hipError_t e = hipEventCreateWithFlags(&copied[l], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&done[l], hipEventDisableTiming);
    if (e == hipSuccess && l >= 2) e = hipStreamWaitEvent(cp, done[l - 2], 0);
    if (e == hipSuccess) e = hipMemcpyAsync(buf, keys_host[l], bytes, hipMemcpyHostToDevice, cp);
    if (e == hipSuccess) e = hipEventRecord(copied[l], cp);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, copied[l], 0);
    if (e != hipSuccess) {
      rc = hip_fail(e, "prefill stream ordering");
      break;
    }
    rc = ls_prefill_index_topk(desc, q_dev[l], w_dev[l], buf, topk_dev[l], ws_dev, ws_bytes,
                               stream);
    if (rc == LS_OK) {
      e = hipEventRecord(done[l], st);
      if (e != hipSuccess) rc = hip_fail(e, "prefill stream ordering");
    }
  }
  // the copy stream ends after the compute stream's last use of the buffers
  if (rc == LS_OK) {
    hipError_t e = hipStreamWaitEvent(cp, done[n_layers - 1], 0);
    if (e != hipSuccess) rc = hip_fail(e, "prefill stream ordering");
  }
  // events still pending are released by the runtime once they complete
  for (int l = 0; l < n_layers; l++) {
    if (copied[l]) (void)hipEventDestroy(copied[l]);
    if (done[l]) (void)hipEventDestroy(done[l]);
  }
  return rc;
}

}  // extern "C"
