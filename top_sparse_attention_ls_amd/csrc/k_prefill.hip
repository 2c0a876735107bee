// Prefill-chunk indexer for gfx950: for every query row of the chunk, the
// scores of all keys it may see (causal), then the per-row top-k.
//
// Method: LeanSparse (arXiv 2611.04671), Abstract -- prefill runs the
// indexer over the layer's whole history; the history is streamed through
// two reusable device buffers so that loading the next layer overlaps the
// current layer's work (ls_prefill_stream_layers in ls_abi.hip).
//
// score[i, t] = sum_h w[i,h] * max(0, q[i,h] . k[t]) for t <= q_pos0 + i,
// computed exactly (int64: with full int8 keys a row can exceed 2^31).
#include "ls_device.h"
#include "ls_launch.h"
#include "ls_bucket.h"

namespace ls {

constexpr int kPrefillRowsPerWG = 2;  // query rows sharing each key tile
constexpr int kPrefillWaves = 8;      // waves of a workgroup, all on its rows

__global__ __launch_bounds__(256) void k_prefill_ctx(int32_t* __restrict__ ctx, int rows,
                                                      int first_pos, int max_ctx) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < rows) ctx[i] = min(max(first_pos + i + 1, 0), max_ctx);
}

// Scores of kPrefillRowsPerWG query rows against every key they may see, as
// an int8 GEMM on v_mfma_i32_16x16x64_i8: A = one row's query (16 heads per
// tile, held in VGPRs), B = 16 keys.  Lane (n, g) holds, for k-step mf,
// dims 32 g + 16 mf .. +15 of head (or key) n: the same dims in A and B, so
// every MFMA contracts 64 of the 128 dims (D = 64: dims 16 g .. +15).
// Epilogue per key: max(., 0) times the head weight (24-bit multiply-add),
// summed over four heads in int32 (< 2^30), then over head tiles in int64,
// then across the four lane groups with a reduce-scatter that leaves one
// key per lane.  Each lane buckets its row's score into that row's LDS
// histogram, the first pass of the selection.  The workgroup owns its rows:
// kPrefillWaves waves stride over the keys (64 per wave step), the query
// operands are loaded once, and the rows' histograms are zeroed once and
// stored whole at the end (no global atomics).  Keys past a row's causal
// limit are computed with the rest of the tile but neither stored nor
// counted.  Key loads are clamped to the last key and ping-pong prefetched
// one workgroup step ahead.
template <int D, int HT>
__global__ __launch_bounds__(64 * kPrefillWaves) void k_prefill_scores(
    const int8_t* __restrict__ q, const int8_t* __restrict__ w, const int8_t* __restrict__ keys,
    int64_t* __restrict__ scores, uint32_t* __restrict__ hist, int rows, int first_pos, int H,
    int max_ctx) {
  constexpr int QR = kPrefillRowsPerWG;
  constexpr int NMF = D / 64;
  __shared__ uint32_t lhist[QR][kWideBins];

  constexpr int NT = 64 * kPrefillWaves;
  const int r0 = blockIdx.x * QR;
  int nv[QR];
  int nv_max = 0;
#pragma unroll
  for (int r = 0; r < QR; r++) {
    nv[r] = (r0 + r < rows) ? min(max(first_pos + r0 + r + 1, 0), max_ctx) : 0;
    nv_max = max(nv_max, nv[r]);
  }
  const int t_end = nv_max;

  for (int i = threadIdx.x; i < QR * kWideBins; i += NT) (&lhist[0][0])[i] = 0;

  const int l = lane_id(), n = l & 15, g = l >> 4;
  const int off = (D == 128) ? 32 * g : 16 * g;
  v4i qa[QR][HT][NMF];
  int32_t wv[QR][HT][4];
#pragma unroll
  for (int r = 0; r < QR; r++) {
    const int row = min(r0 + r, rows - 1);
    const int8_t* qr = q + (size_t)row * H * D;
#pragma unroll
    for (int mt = 0; mt < HT; mt++) {
      // unconditional loads (clamped index, result selected): a load under
      // a divergent condition would be a branch that waits for it
      const int h = 16 * mt + n;
#pragma unroll
      for (int mf = 0; mf < NMF; mf++) {
        const v4i v = *(const v4i*)(qr + (size_t)min(h, H - 1) * D + off + 16 * mf);
        qa[r][mt][mf] = (h < H) ? v : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int hh = 16 * mt + 4 * g + i;
        const int32_t wr = (int32_t)w[(size_t)row * H + min(hh, H - 1)];
        wv[r][mt][i] = hh < H ? wr : 0;
      }
    }
  }
  __syncthreads();

  const int8_t* kb = keys + off;
  const int t_last = t_end - 1;
  auto load4 = [&](int base, v4i (&raw)[4][NMF]) {
#pragma unroll
    for (int tt = 0; tt < 4; tt++) {
      const int t = min(base + 16 * tt + n, t_last);
#pragma unroll
      for (int mf = 0; mf < NMF; mf++) raw[tt][mf] = *(const v4i*)(kb + (size_t)t * D + 16 * mf);
    }
  };
  auto process = [&](int base, const v4i (&raw)[4][NMF]) {
    int64_t part[QR][4];
#pragma unroll
    for (int tt = 0; tt < 4; tt++) {
      v4i acc[QR][HT];
#pragma unroll
      for (int r = 0; r < QR; r++)
#pragma unroll
        for (int mt = 0; mt < HT; mt++)
          acc[r][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[r][mt][0], raw[tt][0],
                                                             v4i{0, 0, 0, 0}, 0, 0, 0);
      if (NMF == 2) {
#pragma unroll
        for (int r = 0; r < QR; r++)
#pragma unroll
          for (int mt = 0; mt < HT; mt++)
            acc[r][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[r][mt][NMF - 1],
                                                               raw[tt][NMF - 1], acc[r][mt], 0,
                                                               0, 0);
      }
#pragma unroll
      for (int r = 0; r < QR; r++) {
        int64_t s = 0;
#pragma unroll
        for (int mt = 0; mt < HT; mt++) {
          int32_t s4 = 0;
#pragma unroll
          for (int i = 0; i < 4; i++) s4 += __mul24(wv[r][mt][i], max(acc[r][mt][i], 0));
          s += (int64_t)s4;
        }
        part[r][tt] = s;
      }
    }
    const int t = base + l;
#pragma unroll
    for (int r = 0; r < QR; r++) {
      // reduce-scatter over the four lane groups: lane (n, g) ends with tile g
      const int64_t score = (int64_t)reduce_scatter4((uint64_t)part[r][0], (uint64_t)part[r][1],
                                                     (uint64_t)part[r][2], (uint64_t)part[r][3]);
      if (t < nv[r]) {
        scores[(size_t)(r0 + r) * max_ctx + t] = score;
        atomicAdd(&lhist[r][wide_bucket(score)], 1u);
      }
    }
  };

  constexpr int S = 64 * kPrefillWaves;  // keys per workgroup step
  int base = __builtin_amdgcn_readfirstlane(wave_id() * 64);
  if (base < t_end) {
    v4i bufA[4][NMF], bufB[4][NMF];
    load4(base, bufA);
    while (true) {
      load4(base + S, bufB);
      __builtin_amdgcn_sched_barrier(0);
      process(base, bufA);
      base += S;
      if (base >= t_end) break;
      load4(base + S, bufA);
      __builtin_amdgcn_sched_barrier(0);
      process(base, bufB);
      base += S;
      if (base >= t_end) break;
    }
  }
  __syncthreads();
  // the rows' histograms are complete: store them whole
#pragma unroll
  for (int r = 0; r < QR; r++) {
    if (r0 + r >= rows) continue;
    uint32_t* hb = hist + (size_t)(r0 + r) * kWideBins;
    for (int i = threadIdx.x; i < kWideBins; i += NT) hb[i] = lhist[r][i];
  }
}

hipError_t launch_prefill_block(const int8_t* q, const int8_t* w, const int8_t* keys,
                                const WideWS& ws, int32_t* ctx, int32_t* topk_out, int rows,
                                int first_pos, int H, int D, int max_ctx, int K, hipStream_t st) {
  hipLaunchKernelGGL(k_prefill_ctx, dim3((rows + 255) / 256), dim3(256), 0, st, ctx, rows,
                     first_pos, max_ctx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((rows + kPrefillRowsPerWG - 1) / kPrefillRowsPerWG);
  const int HT = (H + 15) / 16;
#define LS_PREFILL(DD, TT)                                                                  \
  hipLaunchKernelGGL((k_prefill_scores<DD, TT>), grid, dim3(64 * kPrefillWaves), 0, st, q, w, \
                     keys, ws.scores, ws.hist, rows, first_pos, H, max_ctx)
  if (D == 128) {
    if (HT == 1) LS_PREFILL(128, 1); else if (HT == 2) LS_PREFILL(128, 2);
    else if (HT == 3) LS_PREFILL(128, 3); else LS_PREFILL(128, 4);
  } else {
    if (HT == 1) LS_PREFILL(64, 1); else if (HT == 2) LS_PREFILL(64, 2);
    else if (HT == 3) LS_PREFILL(64, 3); else LS_PREFILL(64, 4);
  }
#undef LS_PREFILL
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_wide_select(ctx, ws, topk_out, rows, max_ctx, K, st);
}

}  // namespace ls
