// Histogram-driven selection for gfx950: keeps the C best scores of every
// row (a decode request's coarse scores, or a prefill query's scores) from
// the per-row bucket histogram that the scoring kernel built.
//
// Method: LeanSparse (arXiv 2611.04671), Abstract -- the coarse pass keeps a
// candidate set that the original indexer keys then refine.
#include <type_traits>

#include "ls_device.h"
#include "ls_select.h"
#include "ls_launch.h"
#include "ls_bucket.h"

namespace ls {

// ------------------------------------------------- candidate select (A2) ----
//
// Keeps the C best tokens under (score desc, position asc), in two kernels
// that meet only at the kernel boundary (the emit workgroups also count
// their arrivals, but only so that the last one clears the tie counter).
//
// k_topc_filter (16384 positions per 1024-thread workgroup): every lane
// first issues its loads -- the request's histogram share, then all 16 of
// its scores (wave w covers 1024 consecutive positions, one coalesced dword
// per lane per wave step, clamped to the row) -- so that the threshold
// search waits only for the histogram.  From the histogram the workgroup
// finds the bucket beta where the count from the top crosses C.  Tokens in
// buckets above beta are kept outright: one wave ballot is one 64-bit word
// of the request's position bitmap, parked in lane u of a register by step u
// and stored by the wave in one piece at the end.  Tokens in bucket beta
// are appended to the wave's own LDS tie list (ranks from the ballot, so no
// atomics in the loop) and the workgroup reserves room in the request's
// global list with one atomic.  Workgroup 0 also stores beta and the count
// above it, and every workgroup its chunk's count of positions kept
// outright, for the emit kernel.
//
// k_topc_emit (one workgroup per filter chunk): resolves the tie list
// exactly and emits its chunk's kept positions at their place in the
// request's ascending list (details at the kernel).

constexpr int kFilterThreads = 1024;
constexpr int kFilterIters = 16;
constexpr int kFilterChunk = kFilterThreads * kFilterIters;  // 16384 positions
constexpr int kFilterWaveTies = 256;

template <class S>
__global__ __launch_bounds__(kFilterThreads) void k_topc_filter(
    const int32_t* __restrict__ ctx_len, const typename S::T* __restrict__ scores,
    const uint32_t* __restrict__ hist, uint32_t* __restrict__ bitmap,
    typename S::T* __restrict__ tie_s, int32_t* __restrict__ tie_p, uint32_t* __restrict__ ctr,
    uint32_t* __restrict__ chunk, int max_ctx, int C, int bitmap_words) {
  using T = typename S::T;
  using U = typename std::make_unsigned<T>::type;
  constexpr int NW = kFilterThreads / kWave;
  constexpr int kPer = (S::kBins + kFilterThreads - 1) / kFilterThreads;
  static_assert(kFilterIters <= kWave / 2, "one bitmap word pair per lane");
  __shared__ uint32_t scan_sh[NW];
  __shared__ int sh_beta;
  __shared__ uint32_t sh_above;
  __shared__ uint32_t wave_n[NW];
  __shared__ uint32_t wave_k[NW];
  __shared__ uint32_t g_base;
  __shared__ T loc_s[NW][kFilterWaveTies];
  __shared__ int32_t loc_p[NW][kFilterWaveTies];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, l = lane_id(), wv = wave_id();
  const int c0 = blockIdx.x * kFilterChunk;
  const int p0 = c0 + wv * (kFilterIters * kWave);  // this wave's first position
  uint32_t* cr = ctr + (size_t)kCtrStride * b;

  const int n_valid = clamp_ctx(ctx_len, b, max_ctx);
  const uint32_t* hb = hist + (size_t)b * S::kBins;
  const int seg = kFilterThreads - 1 - tid;  // thread 0 owns the top bins
  uint32_t hc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; k++) {
    const int bin = seg * kPer + k;
    hc[k] = bin < S::kBins ? hb[bin] : 0u;
  }
  __builtin_amdgcn_sched_barrier(0);
  const T* sb = scores + (size_t)b * max_ctx;
  T sv[kFilterIters];
#pragma unroll
  for (int u = 0; u < kFilterIters; u++) sv[u] = sb[min(p0 + u * kWave + l, max_ctx - 1)];

  // threshold bucket from the histogram
  if (tid == 0) {
    sh_beta = -1;
    sh_above = 0;
  }
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < kPer; k++) s += hc[k];
  uint32_t tot;
  const uint32_t above_seg = block_excl_scan<kFilterThreads>(s, scan_sh, &tot);
  if (n_valid > C && above_seg < (uint32_t)C && (uint32_t)C <= above_seg + s) {
    uint32_t run = above_seg;
#pragma unroll
    for (int k = kPer - 1; k >= 0; k--) {
      if (run < (uint32_t)C && run + hc[k] >= (uint32_t)C) {
        sh_beta = seg * kPer + k;
        sh_above = run;
      }
      run += hc[k];
    }
  }
  __syncthreads();
  const int beta = sh_beta;
  if (blockIdx.x == 0 && tid == 0) {
    cr[kCtrBeta] = (uint32_t)beta;
    cr[kCtrAbove] = sh_above;
  }

  // bucket beta holds the scores [beta_lo, beta_hi]: above it means kept,
  // inside it means tied -- one unsigned compare, (x - beta_lo) < span (no
  // bucket: every valid token is kept and span = 0 admits no tie)
  T beta_lo = 0, beta_hi = 0;
  if (beta >= 0) S::range(beta, beta_lo, beta_hi);
  const bool all_keep = beta < 0;
  const U span = all_keep ? (U)0 : (U)((U)beta_hi - (U)beta_lo) + (U)1;
  const size_t tb = (size_t)b * max_ctx;
  uint32_t wn = 0;     // this wave's ties so far (wave-uniform)
  uint32_t wk = 0;     // this wave's kept positions (wave-uniform)
  uint32_t bw_lo = 0, bw_hi = 0;  // lane u: the bitmap words of step u
#pragma unroll
  for (int u = 0; u < kFilterIters; u++) {
    const int t = p0 + u * kWave + l;
    const bool valid = t < n_valid;
    const bool keep_f = valid & (all_keep | (sv[u] > beta_hi));
    const bool tie_f = valid & ((U)((U)sv[u] - (U)beta_lo) < span);
    const uint64_t mk = __ballot(keep_f);
    const uint64_t mt = __ballot(tie_f);
    bw_lo = l == u ? (uint32_t)mk : bw_lo;
    bw_hi = l == u ? (uint32_t)(mk >> 32) : bw_hi;
    if (mt) {  // wave-uniform
      if (tie_f) {
        const uint32_t idx = wn + lane_rank(mt);
        if (idx < (uint32_t)kFilterWaveTies) {
          loc_s[wv][idx] = sv[u];
          loc_p[wv][idx] = t;
        } else {  // more ties than the wave's LDS list holds: straight to the global list
          const uint32_t g = atomicAdd(&cr[kCtrTies], 1u);
          tie_s[tb + g] = sv[u];
          tie_p[tb + g] = t;
        }
      }
      wn += (uint32_t)__popcll(mt);
    }
    wk += (uint32_t)__popcll(mk);
  }
  // the wave's 32 bitmap words (positions p0 .. p0 + 1023) in one store
  {
    const int w = p0 / 32 + 2 * l;
    if (l < kFilterIters && w < bitmap_words) *(uint2*)&bitmap[(size_t)b * bitmap_words + w] =
        make_uint2(bw_lo, bw_hi);
  }
  if (l == 0) {
    wave_n[wv] = min(wn, (uint32_t)kFilterWaveTies);
    wave_k[wv] = wk;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t n = 0, k = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      n += wave_n[w];
      k += wave_k[w];
    }
    g_base = n ? atomicAdd(&cr[kCtrTies], n) : 0u;  // one reservation per workgroup
    chunk[(size_t)b * gridDim.x + blockIdx.x] = k;  // positions kept outright in this chunk
  }
  __syncthreads();
  uint32_t off = g_base;
  for (int w = 0; w < wv; w++) off += wave_n[w];
  const uint32_t mine = wave_n[wv];
  for (uint32_t i = l; i < mine; i += kWave) {
    tie_s[tb + off + i] = loc_s[wv][i];
    tie_p[tb + off + i] = loc_p[wv][i];
  }
}

constexpr int kEmitThreads = 512;
static_assert(kFilterChunk / 32 == kSelectChunkWords && kSelectChunkWords == kEmitThreads,
              "one filter and one emit workgroup per chunk, one bitmap word per emit thread");

// LDS budget of the emit kernel per score kind: the tie list as
// (order-preserving key, position) entries.
template <class S> struct EmitCfg;
template <> struct EmitCfg<NarrowScore> {
  static constexpr int kTies = 3072;
  using E = uint2;
  static __device__ __forceinline__ E pack(int32_t s, int32_t p) {
    return make_uint2((uint32_t)key_of_i32(s), (uint32_t)p);
  }
  static __device__ __forceinline__ uint64_t key(const E& e) { return e.x; }
  static __device__ __forceinline__ uint32_t pos(const E& e) { return e.y; }
  static __device__ __forceinline__ uint64_t key_of(int32_t s) { return key_of_i32(s); }
};
template <> struct EmitCfg<WideScore> {
  static constexpr int kTies = 4096;
  using E = uint4;
  static __device__ __forceinline__ E pack(int64_t s, int32_t p) {
    const uint64_t k = key_of_i64(s);
    return make_uint4((uint32_t)k, (uint32_t)(k >> 32), (uint32_t)p, 0u);
  }
  static __device__ __forceinline__ uint64_t key(const E& e) {
    return (uint64_t)e.x | ((uint64_t)e.y << 32);
  }
  static __device__ __forceinline__ uint32_t pos(const E& e) { return e.z; }
  static __device__ __forceinline__ uint64_t key_of(int64_t s) { return key_of_i64(s); }
};

// k_topc_emit: one 512-thread workgroup per (request, run of cpw chunks of
// 16384 positions).  With few requests cpw = 1, so a request's emission
// spreads over as many workgroups as its filter; with many (prefill rows)
// one workgroup takes all of a row's chunks.  Every workgroup resolves the
// request's tie list itself (one wave runs the radix threshold search when
// the list fits in LDS, the whole workgroup otherwise): the list is short,
// and repeating the search costs less than another kernel boundary.  Its
// output offset is the kept count of the chunks before its run (written by
// the filter) plus the winning ties before it.  For each chunk of the run it
// sets the winners' bits in an LDS copy of the chunk's 512 bitmap words and
// emits the kept positions in ascending order, one word per thread.  The
// first run pads the list with -1.  Each workgroup clears its share of the
// request's histogram; the last one to finish clears the tie counter.
template <class S>
__global__ __launch_bounds__(kEmitThreads) void k_topc_emit(
    const int32_t* __restrict__ ctx_len, uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ bitmap, const typename S::T* __restrict__ tie_s,
    const int32_t* __restrict__ tie_p, uint32_t* __restrict__ ctr,
    const uint32_t* __restrict__ chunk, int32_t* __restrict__ cand, int max_ctx, int C,
    int bitmap_words, int n_chunks, int cpw) {
  using Cfg = EmitCfg<S>;
  constexpr int NT = kEmitThreads;
  __shared__ uint32_t scan_sh[NT / kWave];
  __shared__ SelectShared ssh;
  __shared__ uint32_t bm_l[kSelectChunkWords];
  __shared__ typename Cfg::E lds_t[Cfg::kTies];  // (key, position) of the ties
  __shared__ Threshold sh_thr;
  __shared__ ThresholdScratch thr_sc;  // the tie search's short list
  const int n_runs = gridDim.x;  // workgroups per request
  // (run, request), numbered so that one request's workgroups share an
  // XCD's L2 (they all read the request's tie list)
  const int lin = xcd_major(blockIdx.x + n_runs * blockIdx.y, n_runs * gridDim.y);
  const int run = lin % n_runs, b = lin / n_runs;
  const int ck0 = run * cpw, ck1 = min(ck0 + cpw, n_chunks);  // this workgroup's chunks
  const int tid = threadIdx.x;
  const int n_valid = clamp_ctx(ctx_len, b, max_ctx);
  const uint32_t* bmg = bitmap + (size_t)b * bitmap_words;
  uint32_t* cr = ctr + (size_t)kCtrStride * b;

  // Issued together, before any of them is waited for: the first kTiePre
  // entries of the tie list (usually all of it; loaded unconditionally,
  // clamped to the row), the run's first bitmap word, the chunk counts
  // before the run and the counters.
  constexpr int kPre = 3;
  constexpr int kTiePre = kPre * NT;
  static_assert(kTiePre <= Cfg::kTies, "the prefetched ties fit the LDS list");
  const typename S::T* ts = tie_s + (size_t)b * max_ctx;
  const int32_t* tp = tie_p + (size_t)b * max_ctx;
  typename S::T ts_pre[kPre];
  int32_t tp_pre[kPre];
#pragma unroll
  for (int k = 0; k < kPre; k++) {
    const int i = min(tid + k * NT, max_ctx - 1);
    ts_pre[k] = ts[i];
    tp_pre[k] = tp[i];
  }
  const uint32_t wd_first = bmg[min(ck0 * kSelectChunkWords + tid, bitmap_words - 1)];
  uint32_t before = 0;  // kept outright in the chunks before the run
  for (int i = tid; i < ck0; i += NT) before += chunk[(size_t)b * n_chunks + i];
  const uint32_t n_tie = cr[kCtrTies];
  const int beta = n_valid > C ? (int)cr[kCtrBeta] : -1;
  const uint32_t above = cr[kCtrAbove];

  uint32_t ties_before = 0;  // winning ties before the run (this thread's share)
  const bool in_lds = n_tie <= (uint32_t)Cfg::kTies;
  // tie i as (order-preserving key, position), from LDS or the global list
  auto tie_entry = [&](int i, uint64_t& u, uint32_t& p) {
    if (in_lds) {
      const typename Cfg::E e = lds_t[i];
      u = Cfg::key(e);
      p = Cfg::pos(e);
    } else {
      u = Cfg::key_of(ts[i]);
      p = (uint32_t)tp[i];
    }
  };
  Threshold thr{0ull, 0u, 0};  // every tie wins when need == n_tie
  if (beta >= 0) {
    const uint32_t need = (uint32_t)C - above;  // 1 <= need <= n_tie
    if (in_lds) {
#pragma unroll
      for (int k = 0; k < kPre; k++) {
        const int i = tid + k * NT;
        if (i < (int)n_tie) lds_t[i] = Cfg::pack(ts_pre[k], tp_pre[k]);
      }
      for (int i = kTiePre + tid; i < (int)n_tie; i += NT) lds_t[i] = Cfg::pack(ts[i], tp[i]);
    }
    __syncthreads();
    if (need < n_tie) {
      if (in_lds) {
        auto get = [&](int i, uint64_t& u, uint32_t& p) {
          const typename Cfg::E e = lds_t[i];
          u = Cfg::key(e);
          p = Cfg::pos(e);
        };
        typename S::T lo, hi;
        S::range(beta, lo, hi);
        thr = tie_threshold<NT>(get, (int)n_tie, need, ssh, &thr_sc, &sh_thr, Cfg::key_of(lo),
                                Cfg::key_of(hi), pos_bits_below(max_ctx));
      } else {
        auto get = [&](int i, uint64_t& u, uint32_t& p) {
          u = Cfg::key_of(ts[i]);
          p = (uint32_t)tp[i];
        };
        thr = block_threshold<NT>(get, (int)n_tie, need, ssh);
      }
    }
    const uint32_t p_lo = 32u * (uint32_t)(ck0 * kSelectChunkWords);
    for (int i = tid; i < (int)n_tie; i += NT) {
      uint64_t u;
      uint32_t p;
      tie_entry(i, u, p);
      if (p < p_lo && keep(thr, u, p)) ties_before++;
    }
  }
  uint32_t base;
  block_excl_scan<NT>(before + ties_before, scan_sh, &base);

  // the run's chunks in order; thread tid owns bitmap word w0 + tid
  int32_t* cb = cand + (size_t)b * C;
  for (int ck = ck0; ck < ck1; ck++) {
    const int w0 = ck * kSelectChunkWords;
    // unconditional load (clamped), selected afterwards; the run's first
    // word was loaded up front
    const uint32_t wd = ck == ck0 ? wd_first : bmg[min(w0 + tid, bitmap_words - 1)];
    bm_l[tid] = w0 + tid < bitmap_words ? wd : 0u;
    __syncthreads();
    if (beta >= 0) {  // the winning ties of this chunk
      const uint32_t p_lo = 32u * (uint32_t)w0, p_hi = p_lo + 32u * kSelectChunkWords;
      for (int i = tid; i < (int)n_tie; i += NT) {
        uint64_t u;
        uint32_t p;
        tie_entry(i, u, p);
        if (p >= p_lo && p < p_hi && keep(thr, u, p))
          atomicOr(&bm_l[(p - p_lo) / 32], 1u << (p % 32));
      }
      __syncthreads();
    }
    const uint32_t word = bm_l[tid];
    uint32_t chunk_total;
    uint32_t off = base + block_excl_scan<NT>((uint32_t)__popc(word), scan_sh, &chunk_total);
    uint32_t bits = word;
    while (bits) {
      const int j = __ffs(bits) - 1;
      if (off < (uint32_t)C) cb[off] = 32 * (w0 + tid) + j;
      off++;
      bits &= bits - 1;
    }
    base += chunk_total;
  }
  // every valid token is kept when there is no threshold bucket; otherwise
  // exactly C are
  if (run == 0) {
    const int total = beta >= 0 ? C : min(n_valid, C);
    for (int i = total + tid; i < C; i += NT) cb[i] = -1;
  }

  // leave the histogram (this workgroup's share) and the tie counter cleared
  uint32_t* hb = hist + (size_t)b * S::kBins;
  const int per = (S::kBins + n_runs - 1) / n_runs;
  for (int i = run * per + tid; i < min((run + 1) * per, S::kBins); i += NT) hb[i] = 0;
  __syncthreads();  // every read of the counters and the tie list is done
  if (tid == 0) {
    if (atomicAdd(&cr[kCtrDone], 1u) == (uint32_t)n_runs - 1) {
      cr[kCtrTies] = 0;
      cr[kCtrDone] = 0;
    }
  }
}

template <class S>
hipError_t launch_emit(const int32_t* ctx_len, const SelectWS<typename S::T>& ws, int32_t* out,
                       int B, int max_ctx, int C, hipStream_t st) {
  const int n_chunks = select_chunks(ws.bitmap_words);
  const int cpw = emit_chunks_per_run(B, n_chunks);
  const dim3 egrid((n_chunks + cpw - 1) / cpw, B);
  hipLaunchKernelGGL(k_topc_emit<S>, egrid, dim3(kEmitThreads), 0, st, ctx_len, ws.hist,
                     ws.bitmap, ws.tie_s, ws.tie_p, ws.ctr, ws.chunk, out, max_ctx, C,
                     ws.bitmap_words, n_chunks, cpw);
  return hipGetLastError();
}

template <class S>
hipError_t launch_select(const int32_t* ctx_len, const SelectWS<typename S::T>& ws, int32_t* out,
                         int B, int max_ctx, int C, hipStream_t st) {
  dim3 grid(select_chunks(ws.bitmap_words), B);
  hipLaunchKernelGGL(k_topc_filter<S>, grid, dim3(kFilterThreads), 0, st, ctx_len, ws.scores,
                     ws.hist, ws.bitmap, ws.tie_s, ws.tie_p, ws.ctr, ws.chunk, max_ctx, C,
                     ws.bitmap_words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_emit<S>(ctx_len, ws, out, B, max_ctx, C, st);
}

hipError_t launch_topc_select(const int32_t* ctx_len, const CoarseWS& ws, int32_t* cand, int B,
                              int max_ctx, int C, hipStream_t st) {
  return launch_select<NarrowScore>(ctx_len, ws, cand, B, max_ctx, C, st);
}

hipError_t launch_wide_select(const int32_t* ctx_len, const WideWS& ws, int32_t* out, int B,
                              int max_ctx, int C, hipStream_t st) {
  return launch_select<WideScore>(ctx_len, ws, out, B, max_ctx, C, st);
}

hipError_t launch_wide_emit(const int32_t* ctx_len, const WideWS& ws, int32_t* out, int B,
                            int max_ctx, int C, hipStream_t st) {
  return launch_emit<WideScore>(ctx_len, ws, out, B, max_ctx, C, st);
}

}  // namespace ls
