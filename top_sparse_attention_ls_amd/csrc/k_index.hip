// Indexer kernels for gfx950: compact-key packing and coarse scoring on int8
// MFMA with a fused score histogram (the candidate selection that consumes
// it is in k_select.hip).
//
// Method: LeanSparse (arXiv 2611.04671), Abstract -- coarse-to-fine indexing
// scores compact key representations and keeps candidates; only those are
// refined with the original indexer keys (k_refine.hip).
#include <hip/hip_ext.h>

#include "ls_device.h"
#include "ls_launch.h"
#include "ls_bucket.h"

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
// whole kernel), the B operand is 16 tokens' compact keys.  This form runs
// requests of up to 16 heads; k_coarse32 below, the same scheme on 32-head
// tiles, runs more.  A stored nibble
// b (two's complement, value v in [-8, 7]) read as b ^ 8 is the offset-binary
// value v + 8 in [0, 15], so one xor and one mask widen it to a byte and the
// MFMA returns dot + c_h with c_h = 8 * sum_d q[h][d]; the query is laid out
// even/odd to match the nibble order.  Then w * max(0, dot) =
// w * max(acc, c_h) - w * c_h: one max and one 24-bit multiply-add per head
// and token, and the constant sum of w * c_h over the lane's heads is
// subtracted once per token.  Sums wrap modulo 2^32, which is exact because
// the true score fits in int32.  The head sum then finishes across the four
// 16-lane groups with a reduce-scatter that leaves one token per lane.
// Every lane then buckets its score into an LDS histogram that is flushed to
// the request's global histogram at the end: the first pass of the
// candidate selection, fused here so that nothing re-reads the scores to
// build it.
//
// Memory: each wave streams 64 tokens (4 KiB of compact keys) per step with
// one 16-byte load per lane per 16-token tile, and prefetches the next 64
// tokens into registers before computing the current ones.  Loads past the
// request's end are clamped to its last token (their results are dropped),
// so the loop has no divergent branches around memory operations.
//
// Exactness: |q.kc| <= 128*128*8 = 2^17, |w| <= 128, 64 heads: |score| <
// 2^31; every partial sum is taken modulo 2^32.

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

// The four 16-token tiles of one 64-token step: lane (n, g) loads token
// base + 16 tt + n (counted from the workgroup's first token) at byte g * LB
// of its row, through a buffer resource over the workgroup's own keys
// (tokens past them read as zero without a memory access, and their scores
// are dropped).  The tile's token offset is a scalar (soffset) and the
// lane's offset a constant, so a load costs no VALU address arithmetic.
template <int D>
__device__ __forceinline__ void coarse_load4(__amdgpu_buffer_rsrc_t kres, uint32_t lane_off,
                                             int base, v4i (&r)[4]) {
  constexpr int KB = D / 2;
#pragma unroll
  for (int tt = 0; tt < 4; tt++) {
    const int so = __builtin_amdgcn_readfirstlane((base + 16 * tt) * KB);
    if (D == 128) {
      r[tt] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(kres, lane_off, so, 0));
    } else {
      const int2 v = __builtin_bit_cast(int2, __builtin_amdgcn_raw_buffer_load_b64(kres, lane_off, so, 0));
      r[tt] = v4i{v.x, v.y, 0, 0};
    }
  }
}

constexpr int kCoarseTileGroup = 2;
constexpr int kCoarseDepth = 2;  // deeper rings measured slower (more bytes in flight)

template <int D, int HT>
__global__ __launch_bounds__(256) void k_coarse(const int8_t* __restrict__ q,
                                                const int8_t* __restrict__ w,
                                                const uint8_t* __restrict__ kc,
                                                const int32_t* __restrict__ ctx_len,
                                                int32_t* __restrict__ scores,
                                                uint32_t* __restrict__ hist, int H,
                                                int max_ctx, int tpw) {
  constexpr int KB = D / 2;       // packed bytes per token
  constexpr int NMF = D / 64;     // MFMAs (K = 64) per head tile
  constexpr int LB = KB / 4;      // bytes per lane per token
  __shared__ uint32_t lhist[kCoarseBins];
  // the workgroup's scores, kept here and written out once at the end: a
  // 4-byte store per lane and step, interleaved with the key stream, costs
  // the key reads far more than one burst of whole 16-byte pieces
  __shared__ __attribute__((aligned(16))) int32_t lsc[kCoarseTokPerWG];

  const int b = blockIdx.y;
  const int n_valid = clamp_ctx(ctx_len, b, max_ctx);
  const int t_begin = blockIdx.x * tpw;
  if (t_begin >= n_valid) return;
  const int t_end = min(t_begin + tpw, n_valid);

  for (int i = threadIdx.x; i < kCoarseBins; i += 256) lhist[i] = 0;

  const int l = lane_id(), n = l & 15, g = l >> 4;
  const int8_t* qb = q + (size_t)b * H * D;
  // c_h = 8 * sum_d q[h][d] of every head, through LDS
  __shared__ int32_t hsum[64];
  if (threadIdx.x < H) {
    const v4i* qh = (const v4i*)(qb + (size_t)threadIdx.x * D);
    int32_t sacc = 0;
#pragma unroll
    for (int j = 0; j < D / 16; j++) {
      const v4i v = qh[j];
#pragma unroll
      for (int k = 0; k < 4; k++) sacc = __builtin_amdgcn_sdot4(v[k], 0x01010101, sacc, false);
    }
    hsum[threadIdx.x] = 8 * sacc;
  }
  v4i qa[HT][NMF];
  int32_t wv[HT][4];
#pragma unroll
  for (int mt = 0; mt < HT; mt++) {
    // unconditional loads from clamped heads, then selected: a load under a
    // divergent condition is a branch that waits for it
    const int h = 16 * mt + n;
    coarse_q_operands<D>(qb + (size_t)min(h, H - 1) * D, g, qa[mt]);
#pragma unroll
    for (int mf = 0; mf < NMF; mf++) qa[mt][mf] = h < H ? qa[mt][mf] : v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int hh = 16 * mt + 4 * g + i;
      const int32_t wr = (int32_t)w[(size_t)b * H + min(hh, H - 1)];
      wv[mt][i] = hh < H ? wr : 0;
    }
  }
  __syncthreads();
  int32_t cv[HT][4];
  uint32_t k_lane = 0;  // sum of w * c_h over this lane's heads
#pragma unroll
  for (int mt = 0; mt < HT; mt++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int hh = 16 * mt + 4 * g + i;
      cv[mt][i] = hh < H ? hsum[hh] : 0;
      k_lane += (uint32_t)(wv[mt][i] * cv[mt][i]);
    }

  // this workgroup's compact keys (tokens past t_end read as zero)
  const __amdgpu_buffer_rsrc_t kres = buffer_rsrc(kc + ((size_t)b * max_ctx + t_begin) * KB,
                                                  (uint32_t)(t_end - t_begin) * KB);
  const uint32_t lane_off = (uint32_t)(n * KB + g * LB);

  // One 64-token step: all MFMAs first (independent accumulators), then the
  // epilogue, so MFMA latency overlaps the VALU work of earlier tiles.
  auto process = [&](int base, const v4i (&raw)[4]) {
    // low / high nibble of every byte as offset binary: (x & m) ^ 8 per byte
    const uint32_t m = 0x0F0F0F0Fu, f = 0x08080808u;
    int32_t part[4];
    // tiles in groups of kCoarseTileGroup: the group's MFMAs, then its
    // epilogue (fewer live accumulators, so more waves fit per SIMD)
#pragma unroll
    for (int t0 = 0; t0 < 4; t0 += kCoarseTileGroup) {
      v4i acc[kCoarseTileGroup][HT];
#pragma unroll
      for (int u = 0; u < kCoarseTileGroup; u++) {
        const int tt = t0 + u;
        const uint32_t x0 = (uint32_t)raw[tt][0], x1 = (uint32_t)raw[tt][1];
        const uint32_t x2 = (uint32_t)raw[tt][2], x3 = (uint32_t)raw[tt][3];
        v4i bop[NMF];
        if (D == 128) {
          bop[0] = v4i{(int)((x0 & m) ^ f), (int)((x1 & m) ^ f), (int)((x2 & m) ^ f),
                       (int)((x3 & m) ^ f)};
          bop[NMF - 1] = v4i{(int)(((x0 >> 4) & m) ^ f), (int)(((x1 >> 4) & m) ^ f),
                             (int)(((x2 >> 4) & m) ^ f), (int)(((x3 >> 4) & m) ^ f)};
        } else {
          bop[0] = v4i{(int)((x0 & m) ^ f), (int)((x1 & m) ^ f), (int)(((x0 >> 4) & m) ^ f),
                       (int)(((x1 >> 4) & m) ^ f)};
        }
#pragma unroll
        for (int mt = 0; mt < HT; mt++)
          acc[u][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[mt][0], bop[0],
                                                             v4i{0, 0, 0, 0}, 0, 0, 0);
        if (NMF == 2) {
#pragma unroll
          for (int mt = 0; mt < HT; mt++)
            acc[u][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[mt][NMF - 1], bop[NMF - 1],
                                                               acc[u][mt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < kCoarseTileGroup; u++) {
        uint32_t s = 0u - k_lane;
#pragma unroll
        for (int mt = 0; mt < HT; mt++)
#pragma unroll
          for (int i = 0; i < 4; i++) s = mad_i24(wv[mt][i], max(acc[u][mt][i], cv[mt][i]), s);
        part[t0 + u] = (int32_t)s;
      }
    }
    const int32_t score = (int32_t)reduce_scatter4((uint32_t)part[0], (uint32_t)part[1],
                                                   (uint32_t)part[2], (uint32_t)part[3]);
    const int t = base + l;
    // no branch: lanes past t_end land on slots that are never written out
    // (or on the last slot, clamped, when the range ends in mid-step, which
    // is then past t_end too), and they add 0 to the histogram
    lsc[min(t - t_begin, kCoarseTokPerWG - 1)] = score;
    atomicAdd(&lhist[coarse_bucket(score)], t < t_end ? 1u : 0u);
  };

  // A ring of kCoarseDepth register buffers: the loads of the next
  // kCoarseDepth - 1 steps are in flight while a step computes.  The main
  // loop runs whole groups of kCoarseDepth steps with a straight-line body
  // (no exit in the middle, so the ring stays in the same registers across
  // the loop edge and nothing drains there); the last steps then use the
  // buffers already loaded.  The scheduling fences keep each step's refill
  // ahead of its compute (the scheduler would otherwise sink it below the
  // wait for the current buffer).
  constexpr int S = 256;  // tokens per workgroup step (4 waves x 64)
  constexpr int R = kCoarseDepth;
  const int base0 = __builtin_amdgcn_readfirstlane(t_begin + wave_id() * 64);
  const int n_steps = base0 < t_end ? (t_end - base0 + S - 1) / S : 0;  // wave-uniform
  if (n_steps > 0) {
    v4i buf[R][4];
#pragma unroll
    for (int k = 0; k < R - 1; k++) coarse_load4<D>(kres, lane_off, base0 - t_begin + k * S, buf[k]);
    int k0 = 0;
    for (; k0 + R <= n_steps; k0 += R) {
#pragma unroll
      for (int j = 0; j < R; j++) {
        coarse_load4<D>(kres, lane_off, base0 - t_begin + (k0 + j + R - 1) * S,
                        buf[(j + R - 1) % R]);
        __builtin_amdgcn_sched_barrier(0);
        process(base0 + (k0 + j) * S, buf[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < R - 1; j++)
      if (k0 + j < n_steps) process(base0 + (k0 + j) * S, buf[j]);
  }
  __syncthreads();
  {
    // the scores: whole 16-byte pieces where the row is 16-byte aligned (it
    // is unless max_ctx is not a multiple of 4), then the rest one by one
    const int n_tok = t_end - t_begin;
    int32_t* sb = scores + (size_t)b * max_ctx + t_begin;
    const int n4 = ((uintptr_t)sb & 15) == 0 ? n_tok / 4 : 0;
    for (int i = threadIdx.x; i < n4; i += 256) *(int4*)(sb + 4 * i) = *(const int4*)&lsc[4 * i];
    for (int j = 4 * n4 + threadIdx.x; j < n_tok; j += 256) sb[j] = lsc[j];
  }
  uint32_t* hb = hist + (size_t)b * kCoarseBins;
  for (int i = threadIdx.x; i < kCoarseBins; i += 256) {
    uint32_t c = lhist[i];
    if (c) atomicAdd(&hb[i], c);
  }
}

// ------------------------------------------- coarse score, 32-head tiles ----
//
// The same scores for more than 16 heads, on v_mfma_i32_32x32x32_i8: one
// instruction does the work of two 16x16x64 ones, and an MFMA instruction
// holds the SIMD's issue for about the same few cycles whatever its size, so
// halving their number leaves more issue to the VALU epilogue beside them
// (at two waves per SIMD, 64 independent VALU operations beside eight
// 16x16x64 MFMAs took 289 ns per iteration, beside four 32x32x32 ones
// 266 ns, and alone 239 ns).
//
// Lane l, t = l % 32, hf = l / 32.  A row t is head 32 mt + t, B column t is
// token 32 tt + t of the wave's 64-token step, and both hold the 16 dims of
// K-slice hf of each K-step: with LB = D / 4 bytes of the packed row per
// half, K-step s of half hf is packed bytes [LB hf + 8 s, +8), widened to
// their 8 low nibbles (even dims) then their 8 high nibbles (odd dims), and
// the query is laid out alike.  D register r of lane l holds head 32 mt +
// 8 (r/4) + 4 hf + r%4 of token t, so a lane's heads give half of its
// token's score and lane l ^ 32 the other half: one 32-lane swap finishes
// both tiles, token l of the step in lane l.  Offsets, exactness and the
// fused histogram are as in k_coarse.
typedef int v16i __attribute__((ext_vector_type(16)));

// Query operand for head row qh, half hf, K-step s: dims [2 (LB hf + 8 s),
// +16), the 8 even ones then the 8 odd ones.
template <int D>
__device__ __forceinline__ v4i coarse32_q_operand(const int8_t* qh, int hf, int s) {
  constexpr int LB = D / 4;
  const v4i a = *(const v4i*)(qh + 2 * (LB * hf + 8 * s));
  const uint32_t w0 = (uint32_t)a[0], w1 = (uint32_t)a[1], w2 = (uint32_t)a[2],
                 w3 = (uint32_t)a[3];
  return v4i{(int)__builtin_amdgcn_perm(w1, w0, 0x06040200u),
             (int)__builtin_amdgcn_perm(w3, w2, 0x06040200u),
             (int)__builtin_amdgcn_perm(w1, w0, 0x07050301u),
             (int)__builtin_amdgcn_perm(w3, w2, 0x07050301u)};
}

template <int D, int HT2>
__global__ __launch_bounds__(256) void k_coarse32(const int8_t* __restrict__ q,
                                                  const int8_t* __restrict__ w,
                                                  const uint8_t* __restrict__ kc,
                                                  const int32_t* __restrict__ ctx_len,
                                                  int32_t* __restrict__ scores,
                                                  uint32_t* __restrict__ hist, int H,
                                                  int max_ctx, int tpw) {
  constexpr int KB = D / 2;   // packed bytes per token
  constexpr int LB = D / 4;   // packed bytes per lane (half a row) per token
  constexpr int NL = LB / 16;  // 16-byte loads per lane per token tile
  constexpr int KS = D / 32;   // K-steps of 32 dims
  static_assert(D == 64 || D == 128, "indexer dim");
  __shared__ uint32_t lhist[kCoarseBins];
  __shared__ __attribute__((aligned(16))) int32_t lsc[kCoarseTokPerWG];

  const int b = blockIdx.y;
  const int n_valid = clamp_ctx(ctx_len, b, max_ctx);
  const int t_begin = blockIdx.x * tpw;
  if (t_begin >= n_valid) return;
  const int t_end = min(t_begin + tpw, n_valid);

  for (int i = threadIdx.x; i < kCoarseBins; i += 256) lhist[i] = 0;

  const int l = lane_id(), t = l & 31, hf = l >> 5;
  const int8_t* qb = q + (size_t)b * H * D;
  // c_h = 8 * sum_d q[h][d] of every head, through LDS
  __shared__ int32_t hsum[64];
  if (threadIdx.x < H) {
    const v4i* qh = (const v4i*)(qb + (size_t)threadIdx.x * D);
    int32_t sacc = 0;
#pragma unroll
    for (int j = 0; j < D / 16; j++) {
      const v4i v = qh[j];
#pragma unroll
      for (int k = 0; k < 4; k++) sacc = __builtin_amdgcn_sdot4(v[k], 0x01010101, sacc, false);
    }
    hsum[threadIdx.x] = 8 * sacc;
  }
  v4i qa[HT2][KS];
  int32_t wv[HT2][16];
#pragma unroll
  for (int mt = 0; mt < HT2; mt++) {
    // unconditional loads from clamped heads, then selected
    const int h = 32 * mt + t;
#pragma unroll
    for (int s = 0; s < KS; s++) {
      const v4i v = coarse32_q_operand<D>(qb + (size_t)min(h, H - 1) * D, hf, s);
      qa[mt][s] = h < H ? v : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int hh = 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
      const int32_t wr = (int32_t)w[(size_t)b * H + min(hh, H - 1)];
      wv[mt][r] = hh < H ? wr : 0;
    }
  }
  __syncthreads();
  int32_t cv[HT2][16];
  uint32_t k_lane = 0;  // sum of w * c_h over this lane's heads
#pragma unroll
  for (int mt = 0; mt < HT2; mt++)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int hh = 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
      cv[mt][r] = hh < H ? hsum[hh] : 0;
      k_lane += (uint32_t)(wv[mt][r] * cv[mt][r]);
    }

  // this workgroup's compact keys (tokens past t_end read as zero)
  const __amdgpu_buffer_rsrc_t kres = buffer_rsrc(kc + ((size_t)b * max_ctx + t_begin) * KB,
                                                  (uint32_t)(t_end - t_begin) * KB);
  const uint32_t lane_off = (uint32_t)(t * KB + hf * LB);
  // the two 32-token tiles of the 64-token step at base (counted from the
  // workgroup's first token): scalar tile offset, constant lane offset
  auto load = [&](int base, v4i (&r)[2][NL]) {
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      const int so = __builtin_amdgcn_readfirstlane((base + 32 * tt) * KB);
#pragma unroll
      for (int i = 0; i < NL; i++)
        r[tt][i] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(kres, lane_off + 16u * i, so, 0));
    }
  };

  // One 64-token step: both tiles' MFMAs, then both epilogues.
  auto process = [&](int base, const v4i (&raw)[2][NL]) {
    const uint32_t m = 0x0F0F0F0Fu, f = 0x08080808u;
    v16i acc[2][HT2];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      uint32_t x[4 * NL];
#pragma unroll
      for (int i = 0; i < NL; i++)
#pragma unroll
        for (int k = 0; k < 4; k++) x[4 * i + k] = (uint32_t)raw[tt][i][k];
#pragma unroll
      for (int s = 0; s < KS; s++) {
        const v4i bop = v4i{(int)((x[2 * s] & m) ^ f), (int)((x[2 * s + 1] & m) ^ f),
                            (int)(((x[2 * s] >> 4) & m) ^ f),
                            (int)(((x[2 * s + 1] >> 4) & m) ^ f)};
#pragma unroll
        for (int mt = 0; mt < HT2; mt++)
          acc[tt][mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              qa[mt][s], bop, s == 0 ? v16i{} : acc[tt][mt], 0, 0, 0);
      }
    }
    uint32_t part[2];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      uint32_t s = 0u - k_lane;
#pragma unroll
      for (int mt = 0; mt < HT2; mt++)
#pragma unroll
        for (int r = 0; r < 16; r++) s = mad_i24(wv[mt][r], max(acc[tt][mt][r], cv[mt][r]), s);
      part[tt] = s;
    }
    // lanes l and l ^ 32 hold the two halves of each token's head sum
    swap32(part[0], part[1]);
    const int32_t score = (int32_t)(part[0] + part[1]);
    const int tok = base + l;
    // no branch: lanes past t_end land on slots that are never written out
    // (or on the last slot, clamped), and they add 0 to the histogram
    lsc[min(tok - t_begin, kCoarseTokPerWG - 1)] = score;
    atomicAdd(&lhist[coarse_bucket(score)], tok < t_end ? 1u : 0u);
  };

  // the register ring of k_coarse (kCoarseDepth buffers, whole groups of
  // steps in a straight-line loop body, the last steps from loaded buffers)
  constexpr int S = 256;  // tokens per workgroup step (4 waves x 64)
  constexpr int R = kCoarseDepth;
  const int base0 = __builtin_amdgcn_readfirstlane(t_begin + wave_id() * 64);
  const int n_steps = base0 < t_end ? (t_end - base0 + S - 1) / S : 0;  // wave-uniform
  if (n_steps > 0) {
    v4i buf[R][2][NL];
#pragma unroll
    for (int k = 0; k < R - 1; k++) load(base0 - t_begin + k * S, buf[k]);
    int k0 = 0;
    for (; k0 + R <= n_steps; k0 += R) {
#pragma unroll
      for (int j = 0; j < R; j++) {
        load(base0 - t_begin + (k0 + j + R - 1) * S, buf[(j + R - 1) % R]);
        __builtin_amdgcn_sched_barrier(0);
        process(base0 + (k0 + j) * S, buf[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < R - 1; j++)
      if (k0 + j < n_steps) process(base0 + (k0 + j) * S, buf[j]);
  }
  __syncthreads();
  {
    const int n_tok = t_end - t_begin;
    int32_t* sb = scores + (size_t)b * max_ctx + t_begin;
    const int n4 = ((uintptr_t)sb & 15) == 0 ? n_tok / 4 : 0;
    for (int i = threadIdx.x; i < n4; i += 256) *(int4*)(sb + 4 * i) = *(const int4*)&lsc[4 * i];
    for (int j = 4 * n4 + threadIdx.x; j < n_tok; j += 256) sb[j] = lsc[j];
  }
  uint32_t* hb = hist + (size_t)b * kCoarseBins;
  for (int i = threadIdx.x; i < kCoarseBins; i += 256) {
    uint32_t c = lhist[i];
    if (c) atomicAdd(&hb[i], c);
  }
}

hipError_t launch_coarse_scores(const int8_t* q, const int8_t* w, const uint8_t* kc,
                                const int32_t* ctx_len, const CoarseWS& ws, int B, int H,
                                int D, int max_ctx, hipStream_t st, hipEvent_t start,
                                hipEvent_t stop) {
  const int tpw = coarse_tokens_per_wg(B, max_ctx);
  dim3 grid((max_ctx + tpw - 1) / tpw, B);
  const bool timed = start != nullptr && stop != nullptr;
#define LS_COARSE(KERN)                                                                      \
  do {                                                                                       \
    if (timed)                                                                               \
      hipExtLaunchKernelGGL(KERN, grid, dim3(256), 0, st, start, stop, 0u, q, w, kc, ctx_len, \
                            ws.scores, ws.hist, H, max_ctx, tpw);                            \
    else                                                                                     \
      hipLaunchKernelGGL(KERN, grid, dim3(256), 0, st, q, w, kc, ctx_len, ws.scores, ws.hist, \
                         H, max_ctx, tpw);                                                   \
  } while (0)
  // up to 16 heads: one 16-head tile; more: 32-head tiles (up to 64 heads)
  if (H <= 16) {
    if (D == 128) LS_COARSE((k_coarse<128, 1>)); else LS_COARSE((k_coarse<64, 1>));
  } else if (H <= 32) {
    if (D == 128) LS_COARSE((k_coarse32<128, 1>)); else LS_COARSE((k_coarse32<64, 1>));
  } else {
    if (D == 128) LS_COARSE((k_coarse32<128, 2>)); else LS_COARSE((k_coarse32<64, 2>));
  }
#undef LS_COARSE
  return hipGetLastError();
}

}  // namespace ls
