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

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its global loads in flight (which __syncthreads()
// would drain).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(256) void k_prefill_ctx(int32_t* __restrict__ ctx, int rows,
                                                      int first_pos, int max_ctx) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < rows) ctx[i] = min(max(first_pos + i + 1, 0), max_ctx);
}

// Scores of kPrefillRowsPerWG query rows against every key they may see, as
// an int8 GEMM on v_mfma_i32_16x16x64_i8, and the first half of their top-k
// selection.  A = one row's query (16 heads per tile, held in VGPRs), B = 16
// keys.  Lane (n, g) holds, for k-step mf, dims 32 g + 16 mf .. +15 of head
// (or key) n: the same dims in A and B, so every MFMA contracts 64 of the
// 128 dims (D = 64: dims 16 g .. +15).  Epilogue per key: max(., 0) times
// the head weight (24-bit multiply-add), summed over eight heads in 32 bits
// (exact: each term is at most 2^28 in magnitude), then in int64, then
// across the four lane groups with a reduce-scatter that leaves one key per
// lane.
//
// The workgroup owns its rows: kPrefillWaves waves stride over the keys (64
// per wave step) with the query operands loaded once, keys ping-pong
// prefetched one workgroup step ahead.  Each score is
// bucketed into its row's LDS histogram and only its bucket (2 bytes) is
// stored -- not the score.  When the keys are done the histogram is
// complete, so the workgroup does the filter's work itself, row by row:
//   - the bucket beta where the count from the top crosses K (none when the
//     row sees at most K keys);
//   - one pass over the row's stored buckets: keys above beta become bitmap
//     bits (one wave ballot per 64 keys), keys in beta are appended to the
//     row's tie list, and every 16384-key chunk's kept count is recorded;
//   - the exact int64 scores of the ties only, recomputed on the MFMA from
//     the query operands still in VGPRs;
//   - the row's counters (tie count, beta, count above beta).
// The emit kernel of the selection then finishes the row.  Keys past a
// row's causal limit are computed with the rest of the tile but neither
// stored nor counted.
template <int D, int HT>
__global__ __launch_bounds__(64 * kPrefillWaves) void k_prefill_select(
    const int8_t* __restrict__ q, const int8_t* __restrict__ w, const int8_t* __restrict__ keys,
    uint16_t* __restrict__ bucket, uint32_t* __restrict__ bitmap, int64_t* __restrict__ tie_s,
    int32_t* __restrict__ tie_p, uint32_t* __restrict__ ctr, uint32_t* __restrict__ chunk,
    int rows, int first_pos, int H, int max_ctx, int K, int bitmap_words) {
  constexpr int QR = kPrefillRowsPerWG;
  constexpr int NMF = D / 64;
  constexpr int NT = 64 * kPrefillWaves;
  constexpr int NW = kPrefillWaves;
  constexpr int kPer = (kWideBins + NT - 1) / NT;  // histogram bins per thread
  constexpr int kChunkIters = kSelectChunkWords * 32 / NT;  // classification steps per chunk
  __shared__ uint32_t lhist[QR][kWideBins];
  __shared__ uint32_t scan_sh[NW];
  __shared__ uint32_t wave_k[NW];
  __shared__ int sh_beta;
  __shared__ uint32_t sh_above;
  __shared__ uint32_t sh_ntie_r[QR];

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

  const int tid = threadIdx.x, l = lane_id(), wv = wave_id(), n = l & 15, g = l >> 4;
  const int off = (D == 128) ? 32 * g : 16 * g;
  v4i qa[QR][HT][NMF];
  int32_t wv4[QR][HT][4];
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
        wv4[r][mt][i] = hh < H ? wr : 0;
      }
    }
  }
  __syncthreads();

  const int8_t* kb = keys + off;
  // scores of 64 keys (lane l: key 16 (l / 16) + l % 16 of the four tiles
  // after the reduce-scatter) for both rows; raw[tt] holds tile tt's keys
  // The tiles are software-pipelined across the two rows: the MFMAs of
  // (row a, tile t) are issued interleaved with the epilogue of the pair
  // before it -- one MFMA, then a share of the other row's max /
  // multiply-adds -- so the matrix core and the VALU work together.  Each
  // row's accumulators are read by the epilogue before that row's next
  // MFMAs overwrite them, so the pipeline needs no extra registers.
  static_assert(QR == 2, "the pipeline alternates two rows");
  auto scores64 = [&](const v4i (&raw)[4][NMF], int64_t (&sc)[QR]) {
    constexpr int NM = HT * NMF;  // MFMAs per (row, tile)
    constexpr int NV = 4 * HT;    // epilogue values per lane per (row, tile)
    v4i acc[QR][HT];
    int64_t part[QR][4];
    auto mfma_i = [&](int r, int tt, int i) {
      const int mt = i % HT, mf = i / HT;
      acc[r][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
          qa[r][mt][mf], raw[tt][mf], mf == 0 ? v4i{0, 0, 0, 0} : acc[r][mt], 0, 0, 0);
    };
    // value j of row r's epilogue: eight heads at a time in 32 bits
    // (|w * relu(dot)| <= 2^28, so a sum of eight lies in [-2^31, 2^31)),
    // then widened
    auto epi_j = [&](int r, int j, uint32_t& s8, int64_t& s) {
      const int mt = j / 4, i = j % 4;
      s8 = mad_i24(wv4[r][mt][i], max(acc[r][mt][i], 0), s8);
      if (j % 8 == 7 || j == NV - 1) {
        s += (int64_t)(int32_t)s8;
        s8 = 0;
      }
    };
#pragma unroll
    for (int i = 0; i < NM; i++) mfma_i(0, 0, i);
#pragma unroll
    for (int k = 1; k < 2 * 4; k++) {
      const int ra = k % 2, ta = k / 2;              // MFMAs of this pair
      const int re = (k - 1) % 2, te = (k - 1) / 2;  // epilogue of the one before
      uint32_t s8 = 0;
      int64_t s = 0;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NM; i++) {
        mfma_i(ra, ta, i);
#pragma unroll
        for (int j = i * NV / NM; j < (i + 1) * NV / NM; j++) epi_j(re, j, s8, s);
        __builtin_amdgcn_sched_barrier(0);
      }
      part[re][te] = s;
    }
    {
      uint32_t s8 = 0;
      int64_t s = 0;
#pragma unroll
      for (int j = 0; j < NV; j++) epi_j(1, j, s8, s);
      part[1][3] = s;
    }
#pragma unroll
    for (int r = 0; r < QR; r++)
      sc[r] = (int64_t)reduce_scatter4((uint64_t)part[r][0], (uint64_t)part[r][1],
                                       (uint64_t)part[r][2], (uint64_t)part[r][3]);
  };

  // ---- scores of every key: buckets stored, histograms in LDS
  // keys through a buffer resource over the ones the rows may see: the
  // tile's key offset is a scalar (soffset), the lane's a constant, and keys
  // past the end read as zero without a memory access (their scores are
  // dropped)
  const __amdgpu_buffer_rsrc_t kres = buffer_rsrc(keys, (uint32_t)t_end * D);
  const uint32_t lane_off = (uint32_t)(n * D + off);
  auto load4 = [&](int base, v4i (&raw)[4][NMF]) {
#pragma unroll
    for (int tt = 0; tt < 4; tt++) {
      const int so = __builtin_amdgcn_readfirstlane((base + 16 * tt) * D);
#pragma unroll
      for (int mf = 0; mf < NMF; mf++)
        raw[tt][mf] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(kres, lane_off + 16 * mf, so, 0));
    }
  };
  auto process = [&](int base, const v4i (&raw)[4][NMF]) {
    int64_t sc[QR];
    scores64(raw, sc);
    const int t = base + l;
#pragma unroll
    for (int r = 0; r < QR; r++) {
      if (t < nv[r]) {
        const uint32_t bk = wide_bucket(sc[r]);
        bucket[(size_t)(r0 + r) * max_ctx + t] = (uint16_t)bk;
        atomicAdd(&lhist[r][bk], 1u);
      }
    }
  };
  constexpr int S = 64 * kPrefillWaves;  // keys per workgroup step
  {
    int base = __builtin_amdgcn_readfirstlane(wv * 64);
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
  }
  __syncthreads();  // every bucket stored, the histograms complete

  // ---- the filter.  Beta of both rows first.
  const int n_chunks = select_chunks(bitmap_words);
  const bool counts = emit_chunks_per_run(rows, n_chunks) == 1;  // the emit reads them
  int beta[QR];
  uint32_t above[QR];
#pragma unroll
  for (int r = 0; r < QR; r++) {
    if (tid == 0) {
      sh_beta = -1;
      sh_above = 0;
    }
    // thread tid holds bins kPer (NT - 1 - tid) .. +kPer-1 (thread 0 the top
    // ones); an exclusive scan gives the count above each segment
    const int seg = NT - 1 - tid;
    uint32_t hc[kPer];
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < kPer; k++) {
      const int bin = seg * kPer + k;
      hc[k] = bin < kWideBins ? lhist[r][bin] : 0u;
      s += hc[k];
    }
    uint32_t tot;
    const uint32_t above_seg = block_excl_scan<NT>(s, scan_sh, &tot);  // (barriers)
    if (nv[r] > K && above_seg < (uint32_t)K && (uint32_t)K <= above_seg + s) {
      uint32_t run = above_seg;
#pragma unroll
      for (int k = kPer - 1; k >= 0; k--) {
        if (run < (uint32_t)K && run + hc[k] >= (uint32_t)K) {
          sh_beta = seg * kPer + k;
          sh_above = run;
        }
        run += hc[k];
      }
    }
    __syncthreads();
    beta[r] = sh_beta;  // -1: every valid key is kept
    above[r] = sh_above;
    __syncthreads();  // sh_beta / sh_above are reused
  }
  if (tid < QR) sh_ntie_r[tid] = 0;
  __syncthreads();

  // One pass over both rows' buckets, a chunk (16384 keys) at a time with the
  // next chunk's buckets in flight: bitmap words (one ballot per 64 keys),
  // tie lists, and -- when the emit reads them -- chunk counts (reduced
  // through LDS behind a barrier that does not wait for the loads in flight).
  auto load_chunk = [&](int ck, uint16_t (&bv)[QR][kChunkIters]) {
#pragma unroll
    for (int r = 0; r < QR; r++) {
      const uint16_t* bb = bucket + (size_t)min(r0 + r, rows - 1) * max_ctx;
#pragma unroll
      for (int it = 0; it < kChunkIters; it++) {
        const int t = (ck * kChunkIters + it) * NT + wv * 64 + l;
        bv[r][it] = bb[min(t, max_ctx - 1)];  // unconditional (clamped), selected below
      }
    }
  };
  auto classify = [&](int ck, const uint16_t (&bv)[QR][kChunkIters]) {
#pragma unroll
    for (int r = 0; r < QR; r++) {
      if (r0 + r >= rows) continue;  // workgroup-uniform
      const int row = r0 + r;
      uint32_t* bm = bitmap + (size_t)row * bitmap_words;
      int32_t* tp = tie_p + (size_t)row * max_ctx;
      uint32_t wk = 0;  // this wave's kept keys in the chunk (wave-uniform)
#pragma unroll
      for (int it = 0; it < kChunkIters; it++) {
        const int base = (ck * kChunkIters + it) * NT + wv * 64;
        const int t = base + l;
        const bool valid = t < nv[r];
        const bool keep_f = valid && (beta[r] < 0 || (int)bv[r][it] > beta[r]);
        const bool tie_f = valid && beta[r] >= 0 && (int)bv[r][it] == beta[r];
        const uint64_t mk = __ballot(keep_f);
        const uint64_t mt = __ballot(tie_f);
        if (l == 0 && base / 32 < bitmap_words)
          *(uint2*)&bm[base / 32] = make_uint2((uint32_t)mk, (uint32_t)(mk >> 32));
        if (mt) {  // wave-uniform
          uint32_t first = 0;
          if (l == 0) first = atomicAdd(&sh_ntie_r[r], (uint32_t)__popcll(mt));
          const uint32_t idx = wave_read(first, 0) + lane_rank(mt);
          if (tie_f) tp[idx] = t;  // idx < nv[r] <= max_ctx
        }
        wk += (uint32_t)__popcll(mk);
      }
      if (counts) {
        if (l == 0) wave_k[wv] = wk;
        lds_barrier();
        if (tid == 0) {
          uint32_t k = 0;
#pragma unroll
          for (int i = 0; i < NW; i++) k += wave_k[i];
          chunk[(size_t)row * n_chunks + ck] = k;
        }
        lds_barrier();
      }
    }
  };
  {
    uint16_t bvA[QR][kChunkIters], bvB[QR][kChunkIters];
    load_chunk(0, bvA);
    for (int ck = 0; ck < n_chunks; ck += 2) {
      if (ck + 1 < n_chunks) load_chunk(ck + 1, bvB);  // workgroup-uniform
      classify(ck, bvA);
      if (ck + 1 >= n_chunks) break;
      if (ck + 2 < n_chunks) load_chunk(ck + 2, bvA);
      classify(ck + 1, bvB);
    }
  }
  __syncthreads();  // tie lists and counts complete (and visible to every wave)

  // exact scores of the ties, 64 per wave step from gathered keys; then the
  // rows' counters
#pragma unroll
  for (int r = 0; r < QR; r++) {
    if (r0 + r >= rows) continue;  // workgroup-uniform
    const int row = r0 + r;
    const uint32_t n_tie = sh_ntie_r[r];
    const int32_t* tp = tie_p + (size_t)row * max_ctx;
    int64_t* ts = tie_s + (size_t)row * max_ctx;
    for (int jb = wv * 64; jb < (int)n_tie; jb += NT) {
      v4i raw[4][NMF];
#pragma unroll
      for (int tt = 0; tt < 4; tt++) {
        const int p = tp[min(jb + 16 * tt + n, (int)n_tie - 1)];
#pragma unroll
        for (int mf = 0; mf < NMF; mf++)
          raw[tt][mf] = *(const v4i*)(kb + (size_t)p * D + 16 * mf);
      }
      int64_t sc[QR];
      scores64(raw, sc);
      if (jb + l < (int)n_tie) ts[jb + l] = sc[r];
    }
    if (tid == 0) {
      uint32_t* cr = ctr + (size_t)kCtrStride * row;
      cr[kCtrTies] = n_tie;
      cr[kCtrBeta] = (uint32_t)beta[r];
      cr[kCtrAbove] = above[r];
    }
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
  hipLaunchKernelGGL((k_prefill_select<DD, TT>), grid, dim3(64 * kPrefillWaves), 0, st, q, w, \
                     keys, ws.bucket, ws.bitmap, ws.tie_s, ws.tie_p, ws.ctr, ws.chunk, rows,  \
                     first_pos, H, max_ctx, K, ws.bitmap_words)
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
  return launch_wide_emit(ctx, ws, topk_out, rows, max_ctx, K, st);
}

}  // namespace ls
