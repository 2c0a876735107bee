// Indexer kernels for gfx950: compact-key packing, coarse scoring on int8
// MFMA with a fused score histogram, and the candidate selection.
//
// Method: LeanSparse (arXiv 2611.04671), Abstract -- coarse-to-fine indexing
// scores compact key representations and keeps candidates; only those are
// refined with the original indexer keys (k_refine.hip).
#include "ls_device.h"
#include "ls_launch.h"

namespace ls {

// ---------------------------------------------------------------- utilities --

__global__ __launch_bounds__(256) void k_fill_zero(uint4* p, size_t n16, uint8_t* tail,
                                                    size_t n_tail) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  size_t stride = (size_t)gridDim.x * 256;
  for (size_t j = i; j < n16; j += stride) p[j] = make_uint4(0, 0, 0, 0);
  if (i < n_tail) tail[i] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  size_t n16 = bytes / 16, n_tail = bytes % 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, st, (uint4*)p, n16,
                     (uint8_t*)p + n16 * 16, n_tail);
  return hipGetLastError();
}

// ------------------------------------------------------------- pack (A0) ----
// kc byte j of a row = (floor(k[2j]/16) & 15) | (floor(k[2j+1]/16) << 4).
// The arithmetic shift of a signed byte is floor division by 16.
__global__ __launch_bounds__(256) void k_pack_coarse(const uint32_t* k8, uint16_t* kc,
                                                      int64_t n_words) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * 256;
  for (; i < n_words; i += stride) {
    uint32_t x = k8[i];  // 4 keys: d = 4i .. 4i+3
    int32_t e0 = (int32_t)(int8_t)(x & 0xFF) >> 4;
    int32_t e1 = (int32_t)(int8_t)((x >> 8) & 0xFF) >> 4;
    int32_t e2 = (int32_t)(int8_t)((x >> 16) & 0xFF) >> 4;
    int32_t e3 = (int32_t)(int8_t)(x >> 24) >> 4;
    uint32_t b0 = (uint32_t)(e0 & 15) | ((uint32_t)(e1 & 15) << 4);
    uint32_t b1 = (uint32_t)(e2 & 15) | ((uint32_t)(e3 & 15) << 4);
    kc[i] = (uint16_t)(b0 | (b1 << 8));
  }
}

hipError_t launch_pack_coarse(const int8_t* k8, uint8_t* kc, int64_t n_rows, int dim,
                              hipStream_t st) {
  // dim is a multiple of 4 (checked by the caller), so rows never split a word.
  int64_t n_words = n_rows * dim / 4;
  int64_t blocks = (n_words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_pack_coarse, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const uint32_t*)k8, (uint16_t*)kc, n_words);
  return hipGetLastError();
}

// ------------------------------------------------------ coarse score (A1) ---
//
// cs[b,t] = sum_h w[b,h] * max(0, sum_d q[b,h,d] * floor(k[b,t,d]/16)).
//
// As an int8 GEMM [heads x D] x [D x tokens] on v_mfma_i32_16x16x64_i8: the
// A operand is the int8 query (16 heads per tile, held in VGPRs for the
// whole kernel), the B operand is 16 tokens' compact keys.  A packed nibble
// n is widened to the byte n*16 by masking (x & 0xF0F0F0F0 for the odd
// elements, (x << 4) & 0xF0F0F0F0 for the even ones), so the MFMA returns
// 16 * dot exactly; the query is laid out even/odd to match.  Epilogue:
// max(.,0) >> 4, times the head weight (24-bit multiply-add), summed over
// heads in-lane and then across the four 16-lane groups with a
// reduce-scatter that leaves one token per lane.  Every lane then buckets its
// score into an LDS histogram that is flushed to the request's global
// histogram at the end: the first pass of the candidate selection, fused
// here so that nothing re-reads the scores to build it.
//
// Memory: each wave streams 64 tokens (4 KiB of compact keys) per step with
// one 16-byte load per lane per 16-token tile, and prefetches the next 64
// tokens into registers before computing the current ones.  Loads past the
// request's end are clamped to its last token (their results are dropped),
// so the loop has no divergent branches around memory operations.
//
// Exactness: |q.kc| <= 128*127*8 < 2^17, |w| <= 128, <= 16 heads per lane
// and 4 lane groups: |sum| < 2^31.

constexpr int kNBHalf = kCoarseBins / 2;

__device__ __forceinline__ uint32_t mag_bucket(uint32_t y) {  // y < 2^31
  if (y < 128u) return y;
  uint32_t e = 31u - (uint32_t)__clz((int)y);
  return 128u + (e - 7u) * 64u + ((y >> (e - 6u)) & 63u);
}

// Monotone bucket of an int32 score in [0, kCoarseBins).
__device__ __forceinline__ uint32_t coarse_bucket(int32_t x) {
  return x >= 0 ? (uint32_t)kNBHalf + mag_bucket((uint32_t)x)
                : (uint32_t)kNBHalf - 1u - mag_bucket((uint32_t)(-(x + 1)));
}

// Query operands for head row qh, lane group g.  D = 128: lane group g owns
// dims [32g, 32g+32); mf 0 holds the even dims, mf 1 the odd ones (byte j =
// dim 32g + 2j + mf).  D = 64: dims [16g, 16g+16); bytes 0..7 the even
// dims, bytes 8..15 the odd ones.
template <int D>
__device__ __forceinline__ void coarse_q_operands(const int8_t* qh, int g, v4i* out) {
  if (D == 128) {
    const v4i a = *(const v4i*)(qh + 32 * g);
    const v4i c = *(const v4i*)(qh + 32 * g + 16);
    const uint32_t w[8] = {(uint32_t)a[0], (uint32_t)a[1], (uint32_t)a[2], (uint32_t)a[3],
                           (uint32_t)c[0], (uint32_t)c[1], (uint32_t)c[2], (uint32_t)c[3]};
    uint32_t ev[4], od[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      ev[k] = __builtin_amdgcn_perm(w[2 * k + 1], w[2 * k], 0x06040200u);
      od[k] = __builtin_amdgcn_perm(w[2 * k + 1], w[2 * k], 0x07050301u);
    }
    out[0] = v4i{(int)ev[0], (int)ev[1], (int)ev[2], (int)ev[3]};
    out[1] = v4i{(int)od[0], (int)od[1], (int)od[2], (int)od[3]};
  } else {
    const v4i a = *(const v4i*)(qh + 16 * g);
    const uint32_t e0 = __builtin_amdgcn_perm((uint32_t)a[1], (uint32_t)a[0], 0x06040200u);
    const uint32_t e1 = __builtin_amdgcn_perm((uint32_t)a[3], (uint32_t)a[2], 0x06040200u);
    const uint32_t o0 = __builtin_amdgcn_perm((uint32_t)a[1], (uint32_t)a[0], 0x07050301u);
    const uint32_t o1 = __builtin_amdgcn_perm((uint32_t)a[3], (uint32_t)a[2], 0x07050301u);
    out[0] = v4i{(int)e0, (int)e1, (int)o0, (int)o1};
  }
}

// Reduce-scatter over the four 16-lane groups: on entry p[tt] is this lane's
// partial for token (tile tt, n); on exit the result is the full sum for
// tile g = lane/16, token n.
template <class T>
__device__ __forceinline__ T reduce_scatter4(T p0, T p1, T p2, T p3, int g) {
  const bool lo = g < 2;
  T s0 = lo ? p2 : p0, s1 = lo ? p3 : p1;
  T r0 = __shfl_xor(s0, 32, kWave), r1 = __shfl_xor(s1, 32, kWave);
  T k0 = (lo ? p0 : p2) + r0;
  T k1 = (lo ? p1 : p3) + r1;
  const bool even = (g & 1) == 0;
  T s = even ? k1 : k0;
  T r = __shfl_xor(s, 16, kWave);
  return (even ? k0 : k1) + r;
}

template <int D>
__device__ __forceinline__ void coarse_load4(const uint8_t* kb, int base, int n, int t_last,
                                             v4i (&r)[4]) {
  constexpr int KB = D / 2;
#pragma unroll
  for (int tt = 0; tt < 4; tt++) {
    const int t = min(base + 16 * tt + n, t_last);
    if (D == 128) {
      r[tt] = *(const v4i*)(kb + (size_t)t * KB);
    } else {
      const int2 v = *(const int2*)(kb + (size_t)t * KB);
      r[tt] = v4i{v.x, v.y, 0, 0};
    }
  }
}

template <int D, int HT>
__global__ __launch_bounds__(256) void k_coarse(const int8_t* __restrict__ q,
                                                const int8_t* __restrict__ w,
                                                const uint8_t* __restrict__ kc,
                                                const int32_t* __restrict__ ctx_len,
                                                int32_t* __restrict__ scores,
                                                uint32_t* __restrict__ hist, int H,
                                                int max_ctx) {
  constexpr int KB = D / 2;       // packed bytes per token
  constexpr int NMF = D / 64;     // MFMAs (K = 64) per head tile
  constexpr int LB = KB / 4;      // bytes per lane per token
  __shared__ uint32_t lhist[kCoarseBins];

  const int b = blockIdx.y;
  const int n_valid = clamp_ctx(ctx_len, b, max_ctx);
  const int t_begin = blockIdx.x * kCoarseTokPerWG;
  if (t_begin >= n_valid) return;
  const int t_end = min(t_begin + kCoarseTokPerWG, n_valid);

  for (int i = threadIdx.x; i < kCoarseBins; i += 256) lhist[i] = 0;

  const int l = lane_id(), n = l & 15, g = l >> 4;
  const int8_t* qb = q + (size_t)b * H * D;
  v4i qa[HT][NMF];
  int32_t wv[HT][4];
#pragma unroll
  for (int mt = 0; mt < HT; mt++) {
    const int h = 16 * mt + n;
    if (h < H) {
      coarse_q_operands<D>(qb + (size_t)h * D, g, qa[mt]);
    } else {
#pragma unroll
      for (int mf = 0; mf < NMF; mf++) qa[mt][mf] = v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int hh = 16 * mt + 4 * g + i;
      wv[mt][i] = hh < H ? (int32_t)w[(size_t)b * H + hh] : 0;
    }
  }
  __syncthreads();

  const uint8_t* kb = kc + (size_t)b * max_ctx * KB + g * LB;
  int32_t* sb = scores + (size_t)b * max_ctx;
  const int t_last = t_end - 1;

  // One 64-token step: all MFMAs first (independent accumulators), then the
  // epilogue, so MFMA latency overlaps the VALU work of earlier tiles.
  auto process = [&](int base, const v4i (&raw)[4]) {
    const uint32_t m = 0xF0F0F0F0u;
    v4i acc[4][HT];
#pragma unroll
    for (int tt = 0; tt < 4; tt++) {
      const uint32_t x0 = (uint32_t)raw[tt][0], x1 = (uint32_t)raw[tt][1];
      const uint32_t x2 = (uint32_t)raw[tt][2], x3 = (uint32_t)raw[tt][3];
      v4i bop[NMF];
      if (D == 128) {
        bop[0] = v4i{(int)((x0 << 4) & m), (int)((x1 << 4) & m), (int)((x2 << 4) & m),
                     (int)((x3 << 4) & m)};
        bop[NMF - 1] = v4i{(int)(x0 & m), (int)(x1 & m), (int)(x2 & m), (int)(x3 & m)};
      } else {
        bop[0] = v4i{(int)((x0 << 4) & m), (int)((x1 << 4) & m), (int)(x0 & m), (int)(x1 & m)};
      }
#pragma unroll
      for (int mt = 0; mt < HT; mt++)
        acc[tt][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[mt][0], bop[0], v4i{0, 0, 0, 0},
                                                            0, 0, 0);
      if (NMF == 2) {
#pragma unroll
        for (int mt = 0; mt < HT; mt++)
          acc[tt][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[mt][NMF - 1], bop[NMF - 1],
                                                              acc[tt][mt], 0, 0, 0);
      }
    }
    int32_t part[4];
#pragma unroll
    for (int tt = 0; tt < 4; tt++) {
      int32_t s = 0;
#pragma unroll
      for (int mt = 0; mt < HT; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) s += __mul24(wv[mt][i], max(acc[tt][mt][i], 0) >> 4);
      part[tt] = s;
    }
    const int32_t score = reduce_scatter4(part[0], part[1], part[2], part[3], g);
    const int t = base + l;
    if (t < t_end) {
      sb[t] = score;
      atomicAdd(&lhist[coarse_bucket(score)], 1u);
    }
  };

  // Ping-pong register buffers: the loads of step i+1 are in flight while
  // step i computes.  Past the end every lane loads row t_last (one line).
  int base = __builtin_amdgcn_readfirstlane(t_begin + wave_id() * 64);
  if (base < t_end) {
    v4i bufA[4], bufB[4];
    coarse_load4<D>(kb, base, n, t_last, bufA);
    while (true) {
      coarse_load4<D>(kb, base + 256, n, t_last, bufB);
      process(base, bufA);
      base += 256;
      if (base >= t_end) break;
      coarse_load4<D>(kb, base + 256, n, t_last, bufA);
      process(base, bufB);
      base += 256;
      if (base >= t_end) break;
    }
  }
  __syncthreads();
  uint32_t* hb = hist + (size_t)b * kCoarseBins;
  for (int i = threadIdx.x; i < kCoarseBins; i += 256) {
    uint32_t c = lhist[i];
    if (c) atomicAdd(&hb[i], c);
  }
}

hipError_t launch_coarse_scores(const int8_t* q, const int8_t* w, const uint8_t* kc,
                                const int32_t* ctx_len, const CoarseWS& ws, int B, int H,
                                int D, int max_ctx, hipStream_t st) {
  dim3 grid((max_ctx + kCoarseTokPerWG - 1) / kCoarseTokPerWG, B);
  const int HT = (H + 15) / 16;
#define LS_COARSE(DD, TT)                                                                  \
  hipLaunchKernelGGL((k_coarse<DD, TT>), grid, dim3(256), 0, st, q, w, kc, ctx_len, ws.scores, \
                     ws.hist, H, max_ctx)
  if (D == 128) {
    if (HT == 1) LS_COARSE(128, 1); else if (HT == 2) LS_COARSE(128, 2);
    else if (HT == 3) LS_COARSE(128, 3); else LS_COARSE(128, 4);
  } else {
    if (HT == 1) LS_COARSE(64, 1); else if (HT == 2) LS_COARSE(64, 2);
    else if (HT == 3) LS_COARSE(64, 3); else LS_COARSE(64, 4);
  }
#undef LS_COARSE
  return hipGetLastError();
}

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
