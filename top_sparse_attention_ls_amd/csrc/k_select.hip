// Candidate selection for gfx950: keeps the C best coarse scores of every
// request from the score histogram the coarse kernel built.
//
// Method: LeanSparse (arXiv 2611.04671), Abstract -- the coarse pass keeps a
// candidate set that the original indexer keys then refine.
#include "ls_device.h"
#include "ls_launch.h"
#include "ls_bucket.h"

namespace ls {

// ------------------------------------------------- candidate select (A2) ----
//
// Keeps the C best tokens under (score desc, position asc), in two kernels.
//
// k_topc_filter (many workgroups per request): every workgroup reads the
// request's bucket histogram and finds the bucket beta where the count from
// the top crosses C.  It then filters its chunk of positions: tokens in
// buckets above beta are kept outright -- a bit in the request's position
// bitmap, written one wave ballot (64 positions) at a time; tokens in bucket
// beta are appended to a tie list (wave ballot + mbcnt ranks, one atomic per
// wave).
//
// k_topc_emit (one 1024-thread workgroup per request): resolves the tie list
// exactly with the block radix threshold search (in LDS when it fits), sets
// the winners' bits, emits the kept positions in ascending order from the
// bitmap, and clears the histogram and tie counter for the next call.

// Finds beta and the count strictly above it from a request's histogram.
// NT threads; result in *beta (-1: every valid token is kept) and *above.
template <int NT>
__device__ void coarse_threshold(const uint32_t* hb, int n_valid, int C, int* beta,
                                 uint32_t* above, uint32_t* scan_sh) {
  constexpr int kPer = (kCoarseBins + NT - 1) / NT;
  if (threadIdx.x == 0) {
    *beta = -1;
    *above = 0;
  }
  __syncthreads();
  if (n_valid <= C) return;
  const int seg = NT - 1 - (int)threadIdx.x;  // thread 0 owns the top segment
  uint32_t s = 0;
  for (int k = 0; k < kPer; k++) {
    const int bin = seg * kPer + k;
    if (bin < kCoarseBins) s += hb[bin];
  }
  uint32_t tot;
  const uint32_t above_seg = block_excl_scan<NT>(s, scan_sh, &tot);
  if (above_seg < (uint32_t)C && (uint32_t)C <= above_seg + s) {
    uint32_t run = above_seg;
    for (int k = kPer - 1; k >= 0; k--) {
      const int bin = seg * kPer + k;
      const uint32_t c = bin < kCoarseBins ? hb[bin] : 0u;
      if (run + c >= (uint32_t)C) {
        *beta = bin;
        *above = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void k_topc_filter(const int32_t* __restrict__ ctx_len,
                                                     const int32_t* __restrict__ scores,
                                                     const uint32_t* __restrict__ hist,
                                                     uint32_t* __restrict__ bitmap,
                                                     int32_t* __restrict__ tie_s,
                                                     int32_t* __restrict__ tie_p,
                                                     uint32_t* __restrict__ ctr, int max_ctx,
                                                     int C, int bitmap_words) {
  __shared__ uint32_t scan_sh[4];
  __shared__ int sh_beta;
  __shared__ uint32_t sh_above;
  __shared__ uint32_t n_local, g_base;
  __shared__ int32_t loc_s[kSelectChunk];
  __shared__ int32_t loc_p[kSelectChunk];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, l = lane_id();
  const int n_valid = clamp_ctx(ctx_len, b, max_ctx);
  if (tid == 0) n_local = 0;
  coarse_threshold<256>(hist + (size_t)b * kCoarseBins, n_valid, C, &sh_beta, &sh_above,
                        scan_sh);
  const int beta = sh_beta;
  uint32_t* bm = bitmap + (size_t)b * bitmap_words;
  const int c0 = blockIdx.x * kSelectChunk;
  const int c1 = min(c0 + kSelectChunk, bitmap_words * 32);
  const int32_t* sb = scores + (size_t)b * max_ctx;
  // keep bits go straight to the bitmap; ties are collected in LDS first
  for (int base = c0 + wave_id() * 64; base < c1; base += 256) {
    const int t = base + l;
    const bool valid = t < n_valid;
    const int32_t s = valid ? sb[t] : 0;
    const int bk = (int)coarse_bucket(s);
    const bool keep_f = valid && (beta < 0 || bk > beta);
    const bool tie_f = valid && beta >= 0 && bk == beta;
    const uint64_t mk = __ballot(keep_f);
    const uint64_t mt = __ballot(tie_f);
    if (l == 0) *(uint2*)&bm[base / 32] = make_uint2((uint32_t)mk, (uint32_t)(mk >> 32));
    if (mt) {
      uint32_t off = 0;
      if (l == 0) off = atomicAdd(&n_local, (uint32_t)__popcll(mt));
      off = __shfl(off, 0, kWave);
      if (tie_f) {
        const uint32_t idx = off + lane_rank(mt);
        loc_s[idx] = s;
        loc_p[idx] = t;
      }
    }
  }
  __syncthreads();
  const uint32_t nl = n_local;
  if (nl == 0) return;
  // one reservation per workgroup in the request's tie list
  if (tid == 0) g_base = atomicAdd(&ctr[kCtrStride * b], nl);
  __syncthreads();
  const size_t gb = (size_t)b * max_ctx + g_base;
  for (uint32_t i = tid; i < nl; i += 256) {
    tie_s[gb + i] = loc_s[i];
    tie_p[gb + i] = loc_p[i];
  }
}

constexpr int kEmitThreads = 1024;
constexpr int kTieLds = 6144;

__global__ __launch_bounds__(kEmitThreads) void k_topc_emit(
    const int32_t* __restrict__ ctx_len, uint32_t* __restrict__ hist,
    uint32_t* __restrict__ bitmap, const int32_t* __restrict__ tie_s,
    const int32_t* __restrict__ tie_p, uint32_t* __restrict__ ctr, int32_t* __restrict__ cand,
    int max_ctx, int C, int bitmap_words) {
  __shared__ uint32_t scan_sh[kEmitThreads / kWave];
  __shared__ int sh_beta;
  __shared__ uint32_t sh_above;
  __shared__ SelectShared ssh;
  __shared__ int32_t lds_s[kTieLds];
  __shared__ int32_t lds_p[kTieLds];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n_valid = clamp_ctx(ctx_len, b, max_ctx);
  uint32_t* hb = hist + (size_t)b * kCoarseBins;
  uint32_t* bm = bitmap + (size_t)b * bitmap_words;
  coarse_threshold<kEmitThreads>(hb, n_valid, C, &sh_beta, &sh_above, scan_sh);
  const int beta = sh_beta;

  if (beta >= 0) {
    const uint32_t n_tie = ctr[kCtrStride * b];
    const uint32_t need = (uint32_t)C - sh_above;  // 1 <= need <= n_tie
    const int32_t* ts = tie_s + (size_t)b * max_ctx;
    const int32_t* tp = tie_p + (size_t)b * max_ctx;
    const bool in_lds = n_tie <= (uint32_t)kTieLds;
    if (in_lds) {
      for (int i = tid; i < (int)n_tie; i += kEmitThreads) {
        lds_s[i] = ts[i];
        lds_p[i] = tp[i];
      }
      __syncthreads();
    }
    const int32_t* ss = in_lds ? lds_s : ts;
    const int32_t* pp = in_lds ? lds_p : tp;
    Threshold thr{0ull, 0u, 0};
    if (need < n_tie) {
      auto get = [&](int i, uint64_t& u, uint32_t& p) {
        u = key_of_i32(ss[i]);
        p = (uint32_t)pp[i];
      };
      thr = block_threshold<kEmitThreads>(get, (int)n_tie, need, ssh);
    }
    for (int i = tid; i < (int)n_tie; i += kEmitThreads) {
      const uint32_t p = (uint32_t)pp[i];
      if (keep(thr, key_of_i32(ss[i]), p)) atomicOr(&bm[p / 32], 1u << (p % 32));
    }
    __syncthreads();
  }

  // emit ascending positions: contiguous word ranges per thread, one scan
  const int nw = (n_valid + 31) / 32;
  const int wpt = (nw + kEmitThreads - 1) / kEmitThreads;
  const int w0 = tid * wpt, w1 = min(w0 + wpt, nw);
  uint32_t cnt = 0;
  for (int wi = w0; wi < w1; wi++)
    cnt += __popc(__hip_atomic_load(&bm[wi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  uint32_t total;
  uint32_t off = block_excl_scan<kEmitThreads>(cnt, scan_sh, &total);
  int32_t* cb = cand + (size_t)b * C;
  for (int wi = w0; wi < w1; wi++) {
    uint32_t bits = __hip_atomic_load(&bm[wi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (bits) {
      const int k = __ffs(bits) - 1;
      if (off < (uint32_t)C) cb[off] = 32 * wi + k;
      off++;
      bits &= bits - 1;
    }
  }
  for (int i = (int)total + tid; i < C; i += kEmitThreads) cb[i] = -1;

  // leave the histogram and tie counter cleared for the next call
  for (int i = tid; i < kCoarseBins; i += kEmitThreads) hb[i] = 0;
  if (tid == 0) ctr[kCtrStride * b] = 0;
}

hipError_t launch_topc_select(const int32_t* ctx_len, const CoarseWS& ws, int32_t* cand, int B,
                              int max_ctx, int C, hipStream_t st) {
  dim3 grid((ws.bitmap_words * 32 + kSelectChunk - 1) / kSelectChunk, B);
  hipLaunchKernelGGL(k_topc_filter, grid, dim3(256), 0, st, ctx_len, ws.scores, ws.hist,
                     ws.bitmap, ws.tie_s, ws.tie_p, ws.ctr, max_ctx, C, ws.bitmap_words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_topc_emit, dim3(B), dim3(kEmitThreads), 0, st, ctx_len, ws.hist,
                     ws.bitmap, ws.tie_s, ws.tie_p, ws.ctr, cand, max_ctx, C, ws.bitmap_words);
  return hipGetLastError();
}

}  // namespace ls
