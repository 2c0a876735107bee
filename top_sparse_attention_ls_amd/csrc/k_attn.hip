// Sparse decode attention for gfx950: each query attends only to the rows
// its indexer selected (related-papers list, dynamic sparse attention
// abstract: a top-k subset of the cached KV bounds each token's reads).
//
//   s_i = scale * q . K_i,  o = sum_i softmax(s)_i V_i,  lse = log-sum-exp(s)
//
// k_attn_mfma  -- latent (MLA-style) layout: one shared row per token, K = the
//                 whole row (qk_dim), V = its first v_dim elements.  bf16
//                 v_mfma_f32_16x16x32_bf16 for Q.K^T and P.V, online softmax
//                 in fp32 (exp2 domain), split over the row list.
// k_attn_valu  -- any head layout (MHA / GQA, small head dims), plain VALU.
// k_combine    -- merges the per-split partials (normalised o, log2-lse);
//                 k_combine_wide, one workgroup per row, when the rows are few.
#include "ls_device.h"
#include "ls_launch.h"

namespace ls {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- MFMA path --
//
// Workgroup = 4 waves x 32 query heads (the 128 heads of a request), one
// request, one split of the row list; one workgroup (one wave per SIMD) per
// CU, which leaves every wave 512 registers: Q stays in VGPRs, the O
// accumulator in AGPRs.  Products use v_mfma_f32_32x32x16_bf16, so every
// LDS byte read feeds 32 heads.
//
// Rows are staged 32 at a time in LDS by the gfx950 global->LDS DMA load
// (global_load_lds_dwordx4: lane L's 16 bytes land at base + 16 L) into a
// ring of NBUF buffers: NBUF-1 tiles stream in while one computes, and no
// VGPRs hold tile data.  Every row is read once per request and split.
//
// LDS tile layout: 16-byte chunk c (dims 8c .. 8c+7) of tile row r sits at
// chunk slot c*32 + (r ^ 8*(c&1)).  DMA instruction k (1 KiB) fills slots
// 64k .. 64k+63, i.e. chunks 2k and 2k+1 of all 32 rows; lane L loads row
// (L&31) ^ 8*(L>>5), chunk 2k + (L>>5).  The row swizzle keeps both reads
// below free of bank conflicts.
//
// 32x32 MFMA layouts (lane l, half = l/32): A holds row l%32, k = 8 half..+7;
// B holds column l%32, k = 8 half..+7; D register r holds row
// 8(r/4) + 4 half + r%4 of column l%32.
//
// S^T = K Q^T: A = tile rows (16 dims per step), B = Q^T (head l%32).  The
// accumulator leaves lane (head n, half) with the scores of rows
// 8j + 4 half + i; its registers 8s..8s+7, converted to bf16, are the B
// operand of step s (rows 16s + 8e' + 4 half + i) of O^T = V^T P^T.  The
// matching A operand -- those 8 rows of one V column -- comes from the same
// tile through the LDS transpose read (ds_read_b64_tr_b16): within a 16-lane
// group, lane j points at row base + j/4, columns 4(j%4) .. +3, and lane i
// receives column i of those 4 rows; two reads (row bases 16s + 4 half and
// +8) give the 8 rows.  O^T lands with the head in the lane, so the online
// softmax stays lane-local (a head's 32 rows sit in lanes l and l+32).
//
// No accumulator rescale in the loop: each head's exponent base is the
// maximum score of its first valid tile (the accumulator is still zero then),
// and later tiles may exceed it by up to 2^64 -- probabilities and sums stay
// far inside the fp32/bf16 range and the final o / l is scale-free.  If a
// head's score ever exceeds its base by more, the workgroup recomputes its
// split with the exact maximum seen in the first pass as the base (so every
// probability is <= 1).  This keeps the 256-value accumulator in AGPRs, out
// of reach of VALU code.
constexpr int kTileR = 32;
constexpr int kAttnWaves = 4;
constexpr int kAttnBufs = 4;
constexpr int kHeadsPerWave = 32;
constexpr float kBaseSlack = 64.f;  // log2 units a score may exceed its head's base

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v4i16 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
}

// Byte offset of (row r, chunk c) in a tile buffer.
__device__ __forceinline__ int tile_off(int r, int c) {
  return (c * kTileR + (r ^ ((c & 1) << 3))) * 16;
}

// Largest row range one workgroup handles (its row ids are staged in LDS).
constexpr int kMaxSplitRows = kAttnMaxSplitRows;

// Workgroup barrier without the release/acquire fences of __syncthreads:
// LDS hazards are handled by the explicit waits at each use, and the empty
// asm statements keep the compiler from moving memory operations across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediates (gfx9 encoding): vmcnt <= N, other counters free.
constexpr int waitcnt_vm(int nvm) { return (nvm & 15) | (7 << 4) | (15 << 8) | ((nvm >> 4) << 14); }
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// Wait until at most `ahead` tiles of this wave's DMA (PER_WAVE instructions
// each) are still in flight.  Immediates must be constants, hence the switch.
template <int PER_WAVE>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  switch (ahead) {
    case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(PER_WAVE)); break;
    case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * PER_WAVE)); break;
    default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * PER_WAVE)); break;
  }
}

// The miss gather folded into the attention (GATHER, pool in device memory).
// Each workgroup copies the selected rows of its own split that missed the
// hot buffer, pool[src[i]] -> hot[rows[i]] (rows[i] being the miss's scratch
// row, or the victim slot a commit gave it), in its prologue.  The first
// NBUF-1 tiles, whose DMA starts before that copy, read their missed rows
// straight from the pool; every later tile reads all its rows from the hot
// buffer, after the copy (a pool spread over the whole history costs the
// tile DMA address-translation misses that the request's compact hot block
// does not).  No workgroup reads rows another one writes.
template <int DQK, int DV, int NBUF, bool GATHER>
__global__ __launch_bounds__(kAttnWaves * 64, 1) void k_attn_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ rows, uint16_t* __restrict__ out, float* __restrict__ lse,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse, int Hq, int K,
    int64_t rows_per_req, int64_t row_stride, float scale_log2, int n_splits,
    int rows_per_split, AttnGather ga) {
  constexpr int NW = kAttnWaves;
  constexpr int QK_STEPS = DQK / 16;
  constexpr int DT = DV / 32;
  constexpr int CH = DQK / 8;              // 16-byte chunks per row
  constexpr int TILE_BYTES = CH * kTileR * 16;
  constexpr int N_DMA = TILE_BYTES / 1024;  // 1 KiB DMA instructions per tile
  constexpr int DMA_PER_WAVE = N_DMA / NW;
  static_assert(CH % 2 == 0 && N_DMA % NW == 0 && NBUF <= 4, "tile layout");
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[NBUF][TILE_BYTES];
  __shared__ int32_t rid_lds[kMaxSplitRows + kTileR];

  // (split, head group, request), numbered so that one request's workgroups
  // run on one XCD and share its query and row ids in that L2
  const int lin = xcd_major(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z),
                            gridDim.x * gridDim.y * gridDim.z);
  const int split = lin % gridDim.x, hg = (lin / gridDim.x) % gridDim.y;
  const int b = lin / (gridDim.x * gridDim.y);
  const int l = lane_id(), w = wave_id();
  const int n = l & 31, half = l >> 5;
  const int h = hg * (kHeadsPerWave * NW) + w * kHeadsPerWave + n;
  const bool h_ok = h < Hq;

  const int i_begin = split * rows_per_split;
  const int i_end = min(i_begin + rows_per_split, K);
  const int n_rows = max(i_end - i_begin, 0);
  const int n_tiles = (n_rows + kTileR - 1) / kTileR;
  const int32_t* rq = rows + (size_t)b * K;
  const int32_t* sq = GATHER ? ga.src + (size_t)b * K : nullptr;
  const uint16_t* kvb = kv + (size_t)b * rows_per_req * row_stride;
  const uint16_t* poolb = GATHER ? ga.pool + (size_t)b * ga.pool_rows * row_stride : nullptr;
  // the tile row this lane loads in every DMA instruction, and its chunk parity
  const int dma_row = (l & 31) ^ (half << 3);
  // row id (and, gathering, pool position) at position i of the split,
  // clamped into the request's list (loads are unconditional; positions
  // past the split are padding)
  auto at = [&](int i) { return min(i_begin + min(i, max(n_rows - 1, 0)), K - 1); };
  auto rid_at = [&](int i) { return rq[at(i)]; };
  auto src_at = [&](int i) { return GATHER ? sq[at(i)] : -1; };
  // What a tile position holds, as one code: >= 0 a hot-buffer row, <= -2 the
  // pool row -(code + 2) of a missed entry, -1 padding (and ids out of range).
  // Gathering, a miss reads the pool in the first NBUF-1 tiles and its hot
  // row (written by the prologue's copy) in the others.
  auto code_of = [&](int i, int32_t r, int32_t sp) {
    const bool r_ok = i < n_rows && r >= 0 && r < rows_per_req;
    if (GATHER && i < n_rows && sp >= 0 && sp < ga.pool_rows &&
        (i < (NBUF - 1) * kTileR || !r_ok))
      return -2 - sp;
    return r_ok ? r : -1;
  };

  // Tile DMA of tile t, this lane's row given by its code (padding loads
  // hot row 0): wave w issues instructions k = w, w + NW, ...  (lds_dma16:
  // the waits on it are the explicit vmcnt waits below)
  auto issue_dma_row = [&](int t, int32_t code) {
    const uint16_t* rowp = kvb + (size_t)(code >= 0 ? code : 0) * row_stride;
    if (GATHER && code <= -2) rowp = poolb + (size_t)(-2 - code) * row_stride;
    const uint8_t* src = (const uint8_t*)rowp + 16 * (2 * w + half);
    const uint32_t dst = lds_addr(&tiles[t % NBUF][0]) + 1024u * w;
#pragma unroll
    for (int j = 0; j < DMA_PER_WAVE; j++) lds_dma16(src + 32 * NW * j, dst + 1024u * NW * j);
  };
  auto issue_dma = [&](int t) { issue_dma_row(t, rid_lds[t * kTileR + dma_row]); };

  // The copy (GATHER).  Wave w owns the split's entries w*64 + lane + 256 k;
  // those that missed go to the wave's compact list (pool row, hot row) in
  // LDS -- in tile buffer NBUF-1, which no DMA fills before the loop -- and
  // the wave copies its list, 16-byte piece p (row p / CH, chunk p % CH) by
  // lane p % 64, kCopyU pieces per lane and round, through buffer resources
  // over the request's pool and hot blocks (a piece past the list gets an
  // offset beyond the block: its load returns zero, its store is dropped).
  constexpr int kRidIters = (kMaxSplitRows + kTileR + NW * 64 - 1) / (NW * 64);
  constexpr int kCopyU = 16;
  constexpr int kListMax = kRidIters * 64;
  static_assert(NW * kListMax * 8 <= TILE_BYTES, "copy lists fit a tile buffer");
  int32_t* cl_src = (int32_t*)&tiles[NBUF - 1][0] + w * 2 * kListMax;
  int32_t* cl_dst = cl_src + kListMax;
  int m_list = 0;  // wave-uniform
  uint4 cp_v[kCopyU];
  const uint32_t pool_block = GATHER ? (uint32_t)(ga.pool_rows * row_stride * 2) : 0u;
  const uint32_t hot_block = GATHER ? (uint32_t)(rows_per_req * row_stride * 2) : 0u;
  const uint32_t row_bytes = (uint32_t)(row_stride * 2);
  auto copy_load = [&](int p0) {
    const __amdgpu_buffer_rsrc_t pres = buffer_rsrc(poolb, pool_block);
#pragma unroll
    for (int u = 0; u < kCopyU; u++) {
      const int p = p0 + l + 64 * u;
      const int e = min(p / CH, max(m_list - 1, 0));
      const uint32_t off =
          p < m_list * CH ? (uint32_t)cl_src[e] * row_bytes + 16u * (p - (p / CH) * CH)
                          : pool_block;
      cp_v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pres, off, 0, 0));
    }
  };
  auto copy_store = [&](int p0) {
    const __amdgpu_buffer_rsrc_t hres = buffer_rsrc(kvb, hot_block);
#pragma unroll
    for (int u = 0; u < kCopyU; u++) {
      const int p = p0 + l + 64 * u;
      const int e = min(p / CH, max(m_list - 1, 0));
      const uint32_t off =
          p < m_list * CH ? (uint32_t)cl_dst[e] * row_bytes + 16u * (p - (p / CH) * CH)
                          : hot_block;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, cp_v[u]), hres, off, 0, 0);
    }
  };

  // Prologue in two round trips.  First the query (which needs no row id),
  // each lane's own DMA rows of the first tiles and the split's row ids (to
  // be staged in LDS) -- with their pool positions, gathering; the first
  // tiles' DMA then starts at once, with the copy's pool reads beside it.
  // The query (147 KB per workgroup at 128 heads of 576 dims) thus comes in
  // while the row ids are awaited rather than competing with the first tiles.
  // B operand of S^T = K Q^T: head n, dims 16 ks + 8 half .. +7 (loaded
  // unconditionally from a clamped head, then selected)
  v8bf qB[QK_STEPS];
  {
    const uint16_t* qh = q + ((size_t)b * Hq + min(h, Hq - 1)) * DQK + 8 * half;
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ks++) {
      const v8u16 v = *(const v8u16*)(qh + 16 * ks);
      qB[ks] = __builtin_bit_cast(v8bf, h_ok ? v : v8u16{0, 0, 0, 0, 0, 0, 0, 0});
    }
  }
  int32_t rv[kRidIters], sv[kRidIters];
  {
    int32_t r0[NBUF - 1], s0[NBUF - 1];
#pragma unroll
    for (int t = 0; t < NBUF - 1; t++) {
      r0[t] = rid_at(t * kTileR + dma_row);
      s0[t] = src_at(t * kTileR + dma_row);
    }
#pragma unroll
    for (int k = 0; k < kRidIters; k++) {
      rv[k] = rid_at(threadIdx.x + k * NW * 64);
      sv[k] = src_at(threadIdx.x + k * NW * 64);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
#pragma unroll
    for (int t = 0; t < NBUF - 1; t++)
      if (t < n_tiles) issue_dma_row(t, code_of(t * kTileR + dma_row, r0[t], s0[t]));
  }
  __builtin_amdgcn_sched_barrier(0);
  if (GATHER) {
#pragma unroll
    for (int k = 0; k < kRidIters; k++) {
      const int i = threadIdx.x + k * NW * 64;
      const bool miss = i < n_rows && sv[k] >= 0 && sv[k] < ga.pool_rows && rv[k] >= 0 &&
                        rv[k] < rows_per_req;
      const uint64_t mask = __ballot(miss);
      if (miss) {
        const int e = m_list + (int)lane_rank(mask);
        cl_src[e] = sv[k];
        cl_dst[e] = rv[k];
      }
      m_list += __popcll(mask);
    }
    if (m_list > 0) copy_load(0);
  }
  // Everything has landed (the first tiles too) before the loop, so the
  // compiler has no load of its own outstanding there (it would otherwise
  // wait on every iteration, which would also drain the tile DMA in flight);
  // the loop then waits for each tile's DMA alone.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  if (GATHER && m_list > 0) {
    // the copy's first round has landed: store it; further rounds (more than
    // kCopyU * 64 / CH misses in a wave's 64 entries) one round trip each
    copy_store(0);
    for (int p0 = 64 * kCopyU; p0 < m_list * CH; p0 += 64 * kCopyU) {
      copy_load(p0);
      copy_store(p0);
    }
  }
#pragma unroll
  for (int k = 0; k < kRidIters; k++) {
    const int i = threadIdx.x + k * NW * 64;
    if (i < n_tiles * kTileR) rid_lds[i] = code_of(i, rv[k], sv[k]);
  }
  __shared__ int redo;
  if (threadIdx.x == 0) redo = 0;
  __syncthreads();  // row ids staged

  v16f oacc[DT];
  float m_used, l_run, m_seen = -INFINITY;
  bool over = false;

  // Per-lane LDS byte offsets; every read below is base + compile-time step.
  // QK A operand: row n, chunk 2 ks + half (parity = half): 1024 B per ks.
  const int qk_off = tile_off(n, half);
  // transpose read: 16-lane group G = l/16 covers columns 16 (G&1) .. +15 of
  // a 32-dim tile; lane j = l%16 -> row 16 s + 4 half + j/4 (+8), chunk
  // 4 dt + 2 (G&1) + (j%4)/2, byte 8 (j&1): 2048 B per dt, 256 B per s.
  const int j16 = l & 15, cb = (l >> 4) & 1, par = (j16 & 3) >> 1;
  const int tr_off0 = (2 * cb + par) * 512 + (((4 * half + (j16 >> 2)) ^ (par << 3)) * 16) +
                      8 * (j16 & 1);
  const int tr_off1 = (2 * cb + par) * 512 + (((4 * half + (j16 >> 2) + 8) ^ (par << 3)) * 16) +
                      8 * (j16 & 1);

  // pass 0: base = first valid tile's max; pass 1 (only if a score overran
  // its base by more than kBaseSlack): base = the exact max from pass 0
  for (int pass = 0; pass < 2; pass++) {
  if (pass == 1) {
    if (!redo) break;
    m_used = m_seen;
  } else {
    m_used = -INFINITY;
  }
#pragma unroll
  for (int dt = 0; dt < DT; dt++) oacc[dt] = v16f{};
  l_run = 0.f;
  if (pass == 1)  // pass 0's first tiles were issued with the prologue
    for (int t = 0; t < NBUF - 1 && t < n_tiles; t++) issue_dma(t);
  for (int t = 0; t < n_tiles; t++) {
    // refill the buffer freed at the end of the previous step
    if (t + NBUF - 1 < n_tiles) issue_dma(t + NBUF - 1);
    // loads complete in order: at most `ahead` later tiles still in flight
    wait_tiles_ahead<DMA_PER_WAVE>(min(n_tiles - 1 - t, NBUF - 1));
    wg_barrier();  // tile t is in LDS for every wave
    const uint8_t* cur = &tiles[t % NBUF][0];
    const uint32_t vmask =
        (uint32_t)__ballot(l < kTileR && rid_lds[t * kTileR + (l & 31)] != -1);

    // S^T = K Q^T (32 rows x 32 heads): operand reads run 4 steps ahead of
    // their MFMAs, all on one accumulator.  Back-to-back MFMAs on one AGPR
    // accumulator measured faster here than two alternating ones, and a
    // second chain would cost 16 registers the wave does not have (at 512
    // the kernel spills).
    v16f sacc = {};
    {
      v8u16 ab[4];
#pragma unroll
      for (int i = 0; i < 4; i++) ab[i] = *(const v8u16*)(cur + qk_off + 1024 * i);
#pragma unroll
      for (int ks = 0; ks < QK_STEPS; ks++) {
        const v8u16 a = ab[ks & 3];
        if (ks + 4 < QK_STEPS) ab[ks & 3] = *(const v8u16*)(cur + qk_off + 1024 * (ks + 4));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), qB[ks], sacc,
                                                       0, 0, 0);
      }
      // scheduling contract for the loop above: 4 reads, then MFMA/read pairs
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < QK_STEPS - 4; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    // phase fences for the scheduler: keep the PV operand reads from being
    // hoisted over QK and the softmax, where they would starve QK of VGPRs
    __builtin_amdgcn_sched_barrier(0);
    float sv[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r++) sv[r] = sacc[r] * scale_log2;
    if (vmask != 0xFFFFFFFFu) {  // only a split's last tile can be partial
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = 8 * (r >> 2) + 4 * half + (r & 3);
        sv[r] = ((vmask >> row) & 1u) ? sv[r] : -INFINITY;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; r++) tmax = fmaxf(tmax, sv[r]);
    {
      float lo, hi;  // the head's two 16-row halves (lanes n and n + 32)
      pair32(tmax, lo, hi);
      tmax = fmaxf(lo, hi);
    }
    m_seen = fmaxf(m_seen, tmax);
    if (m_used == -INFINITY) m_used = tmax;         // first valid tile of this head
    else over = over || (tmax > m_used + kBaseSlack);  // never in pass 1
    const float m_ref = (m_used == -INFINITY) ? 0.f : m_used;
    v8bf pB[2];
    {
      uint16_t pb[16];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const float p = __builtin_amdgcn_exp2f(sv[r] - m_ref);  // exp2(-inf) = 0
        psum += p;
        pb[r] = f32_to_bf16_rne(p);
      }
      l_run += psum;
      const v8u16 p0 = {pb[0], pb[1], pb[2], pb[3], pb[4], pb[5], pb[6], pb[7]};
      const v8u16 p1 = {pb[8], pb[9], pb[10], pb[11], pb[12], pb[13], pb[14], pb[15]};
      pB[0] = __builtin_bit_cast(v8bf, p0);
      pB[1] = __builtin_bit_cast(v8bf, p1);
    }
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T P^T, two 16-row steps per 32-dim tile; the transpose reads
    // of tile dt+1 are issued before the MFMAs of tile dt
    {
      auto tr_read = [&](int dt, int ss) {
        const v4i16 a0 = lds_read_tr16(cur + tr_off0 + 2048 * dt + 256 * ss);
        const v4i16 a1 = lds_read_tr16(cur + tr_off1 + 2048 * dt + 256 * ss);
        const v8u16 a = {(uint16_t)a0[0], (uint16_t)a0[1], (uint16_t)a0[2], (uint16_t)a0[3],
                         (uint16_t)a1[0], (uint16_t)a1[1], (uint16_t)a1[2], (uint16_t)a1[3]};
        return a;
      };
      v8u16 va0 = tr_read(0, 0), va1 = tr_read(0, 1);
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
        const v8u16 c0 = va0, c1 = va1;
        if (dt + 1 < DT) {
          va0 = tr_read(dt + 1, 0);
          va1 = tr_read(dt + 1, 1);
        }
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, c0), pB[0],
                                                           oacc[dt], 0, 0, 0);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, c1), pB[1],
                                                           oacc[dt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
      for (int i = 0; i < DT - 1; i++) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    wg_barrier();  // every wave is done reading `cur` before it is refilled
  }
  if (pass == 0) {
    if (over) redo = 1;
    __syncthreads();
  }
  }

  float l_lo, l_hi;
  pair32(l_run, l_lo, l_hi);
  const float l_tot = l_lo + l_hi;
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  const float lse2 = any ? m_used + log2f(l_tot) : -INFINITY;
  // Output rows go through LDS (the tile ring is free: the loop ended with a
  // barrier after the last tile): each wave writes its 32 heads' rows as
  // bf16 into its own region, then stores them whole, 16 bytes per lane, so
  // every store instruction covers one contiguous 1 KiB row.
  // lane (head n, half): oacc[dt][r] = O[head][32 dt + 8 (r/4) + 4 half + r%4]
  constexpr int kRowPitch = DV * 2 + 16;  // bytes; padding spreads the banks
  static_assert(NW * kHeadsPerWave * kRowPitch <= NBUF * TILE_BYTES, "epilogue staging");
  uint8_t* stage = &tiles[0][0] + w * (kHeadsPerWave * kRowPitch);
#pragma unroll
  for (int dt = 0; dt < DT; dt++)
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      uint2 v;
      v.x = (uint32_t)f32_to_bf16_rne(oacc[dt][4 * jj] * inv) |
            ((uint32_t)f32_to_bf16_rne(oacc[dt][4 * jj + 1] * inv) << 16);
      v.y = (uint32_t)f32_to_bf16_rne(oacc[dt][4 * jj + 2] * inv) |
            ((uint32_t)f32_to_bf16_rne(oacc[dt][4 * jj + 3] * inv) << 16);
      *(uint2*)(stage + n * kRowPitch + 2 * (32 * dt + 8 * jj + 4 * half)) = v;
    }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this wave's rows are staged
  static_assert(DV * 2 == 64 * 16, "one 16-byte piece per lane per row");
  const int h0 = hg * (kHeadsPerWave * NW) + w * kHeadsPerWave;
#pragma unroll 4
  for (int hr = 0; hr < kHeadsPerWave; hr++) {
    const int head = h0 + hr;
    if (head >= Hq) break;  // wave-uniform
    const uint4 piece = *(const uint4*)(stage + hr * kRowPitch + 16 * l);
    uint16_t* dst = (n_splits == 1)
                        ? out + ((size_t)b * Hq + head) * DV
                        : part_o + (((size_t)b * Hq + head) * n_splits + split) * DV;
    *(uint4*)((uint8_t*)dst + 16 * l) = piece;
  }
  if (h_ok && half == 0) {
    if (n_splits == 1)
      lse[(size_t)b * Hq + h] = any ? lse2 * kLn2 : -INFINITY;
    else
      part_lse[((size_t)b * Hq + h) * n_splits + split] = lse2;
  }
}

// ---------------------------------------------------------------- VALU path --
// One workgroup per (query head, request), for any head layout (MHA / GQA,
// head dims up to kValuMaxDim).  Scores: every thread takes whole rows (row
// i = tid + 256 k) and loads each row's head slice with 16-byte loads, all of
// them issued before any is used, so the whole score phase costs one round
// trip (the query, staged in LDS as fp32, is read by every thread); block
// max and sum, then P.V with the threads over (row group, 8-dim chunk), the V
// chunk loads of a thread again issued together (the row ids staged in LDS
// by the score phase).  dqk, dv and both strides are multiples of 8 (the
// 16-byte pieces).
constexpr int kValuMaxRows = 8192;
constexpr int kValuMaxDim = 1024;
constexpr int kValuRowsPerThread = kValuMaxRows / 256;

__device__ __forceinline__ float block_reduce_max(float v, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  if (lane_id() == 0) sh[wave_id()] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_reduce_sum(float v, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  if (lane_id() == 0) sh[wave_id()] = v;
  __syncthreads();
  float r = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return r;
}

// dot of the fp32 query in LDS with a row's head slice, 8 dims per piece
__device__ __forceinline__ float dot8(const float* qs, int d0, uint4 v) {
  const uint32_t x[4] = {v.x, v.y, v.z, v.w};
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    acc = fmaf(qs[d0 + 2 * e], __uint_as_float(x[e] << 16), acc);
    acc = fmaf(qs[d0 + 2 * e + 1], __uint_as_float(x[e] & 0xFFFF0000u), acc);
  }
  return acc;
}

template <int DP>  // 16-byte pieces of the score head slice handled per row at once
__global__ __launch_bounds__(256) void k_attn_valu(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kbase,
    const uint16_t* __restrict__ vbase, const int32_t* __restrict__ rows,
    uint16_t* __restrict__ out, float* __restrict__ lse, int Hq, int n_kv, int dqk, int dv,
    int K, int64_t rows_per_req, int64_t row_stride, int64_t head_stride, float scale) {
  __shared__ float qs[kValuMaxDim];
  __shared__ float sc[kValuMaxRows];
  __shared__ int32_t rid_sh[kValuMaxRows];
  __shared__ float red[4];
  __shared__ float acc_sh[256 * 8];
  const int h = blockIdx.x, b = blockIdx.y;
  const int kvh = h / (Hq / n_kv);
  const int tid = threadIdx.x;
  const uint16_t* qh = q + ((size_t)b * Hq + h) * dqk;
  for (int d = tid; d < dqk; d += 256) qs[d] = bf16_to_f32(qh[d]);
  const int32_t* rb = rows + (size_t)b * K;
  const size_t req_off = (size_t)b * rows_per_req * row_stride + (size_t)kvh * head_stride;
  // this thread's rows (ids loaded together; out-of-range ids are padding)
  int32_t r_of[kValuRowsPerThread];
  const int my_rows = K > tid ? (K - 1 - tid) / 256 + 1 : 0;
#pragma unroll
  for (int k = 0; k < kValuRowsPerThread; k++) {
    const int i = tid + 256 * k;
    const int32_t r0 = k < my_rows ? rb[i] : -1;
    r_of[k] = (r0 >= 0 && r0 < rows_per_req) ? r0 : -1;
  }
  __syncthreads();  // query staged
  const int n_pc = dqk / 8;
  float m_loc = -INFINITY;
#pragma unroll 1
  for (int k = 0; k < my_rows; k++) {
    const int32_t r = r_of[k];
    const uint4* kr = (const uint4*)(kbase + req_off + (size_t)(r >= 0 ? r : 0) * row_stride);
    float dot = 0.f;
    for (int c0 = 0; c0 < n_pc; c0 += DP) {
      uint4 v[DP];
#pragma unroll
      for (int u = 0; u < DP; u++) v[u] = kr[min(c0 + u, n_pc - 1)];
#pragma unroll
      for (int u = 0; u < DP; u++)
        if (c0 + u < n_pc) dot += dot8(qs, 8 * (c0 + u), v[u]);
    }
    const float s_ = (r >= 0) ? dot * scale : -INFINITY;
    sc[tid + 256 * k] = s_;
    rid_sh[tid + 256 * k] = r;
    m_loc = fmaxf(m_loc, s_);
  }
  const float m = block_reduce_max(m_loc, red);
  float lsum = 0.f;
  if (m != -INFINITY) {
    for (int k = 0; k < my_rows; k++) {
      const int i = tid + 256 * k;
      const float p = (sc[i] == -INFINITY) ? 0.f : expf(sc[i] - m);
      sc[i] = p;
      lsum += p;
    }
  }
  lsum = block_reduce_sum(lsum, red);  // (its barriers also publish sc)
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* ob = out + ((size_t)b * Hq + h) * dv;
  // P.V: thread (row group rg, 8-dim chunk c); chunks of at most 256 / groups
  const int n_vc = dv / 8;
  const int groups = max(256 / n_vc, 1);
  for (int c0 = 0; c0 < n_vc; c0 += 256) {
    const int nc = min(256, n_vc - c0);
    const int grp = max(256 / nc, 1);
    const int c = c0 + tid % nc, rg = tid / nc;
    float a8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (rg < grp && m != -INFINITY) {
      for (int i0 = rg; i0 < K; i0 += 4 * grp) {
        uint4 v[4];
        float pw[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int i = i0 + grp * u;
          const int32_t r0 = i < K ? rid_sh[i] : -1;   // -1: padding or out of range
          pw[u] = r0 >= 0 ? sc[i] : 0.f;
          v[u] = *((const uint4*)(vbase + req_off + (size_t)(r0 >= 0 ? r0 : 0) * row_stride) + c);
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 4; e++) {
            a8[2 * e] = fmaf(pw[u], __uint_as_float(x[e] << 16), a8[2 * e]);
            a8[2 * e + 1] = fmaf(pw[u], __uint_as_float(x[e] & 0xFFFF0000u), a8[2 * e + 1]);
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) acc_sh[tid * 8 + e] = (rg < grp) ? a8[e] : 0.f;
    __syncthreads();
    if (tid < nc * 8) {
      const int cc = tid / 8, e = tid % 8;
      float tot = 0.f;
      for (int g = 0; g < grp; g++) tot += acc_sh[(g * nc + cc) * 8 + e];
      ob[8 * (c0 + cc) + e] = f32_to_bf16_rne(tot * inv);
    }
    __syncthreads();
  }
  (void)groups;
  if (tid == 0) lse[(size_t)b * Hq + h] = (lsum > 0.f) ? m + logf(lsum) : -INFINITY;
}

// ------------------------------------------------------------------ combine --
// out = sum_j o_j 2^(lse_j - L) with L = log2 sum_j 2^lse_j; lse = L ln 2.
// One wave per (request, head), four per workgroup, numbered like the
// attention grid so that a request's partials are read on the XCD that wrote
// them.  Each lane combines 8 consecutive dims, eight splits at a time.  The
// split LSEs are read eight at a time (L by a running max and rescaled sum),
// and the first CB batches of them and of the partials -- for 512 dims and up
// to 8 CB splits, all of the data -- load together: one round trip per head.
// CB = 1 for up to eight splits; with more (few requests, many splits each)
// CB = 4, so that 32 splits take one round trip instead of a chain of them
// (a separate instance: its 128 registers of partials would cut the
// occupancy of the many-request launches).  DV is a multiple of 8.
template <int CB>
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ part_o,
                                                 const float* __restrict__ part_lse,
                                                 uint16_t* __restrict__ out,
                                                 float* __restrict__ lse, int BH, int DV,
                                                 int n_splits) {
  const int bh = __builtin_amdgcn_readfirstlane(xcd_major(blockIdx.x, gridDim.x) * 4 + wave_id());
  if (bh >= BH) return;
  const int l = lane_id();
  const float* pl = part_lse + (size_t)bh * n_splits;
  const uint16_t* po = part_o + (size_t)bh * n_splits * DV;
  // splits j0 .. j0+7 of dims d .. d+7, and their LSEs (unconditional loads:
  // split and dim clamped; splits past the end get LSE -inf, weight 0)
  auto load8 = [&](int j0, int d, uint4 (&v)[8]) {
    const int dc = min(d, DV - 8);
#pragma unroll
    for (int u = 0; u < 8; u++) v[u] = *(const uint4*)(po + (size_t)min(j0 + u, n_splits - 1) * DV + dc);
  };
  auto load_lse8 = [&](int j0, float (&x)[8]) {
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const float y = pl[min(j0 + u, n_splits - 1)];
      x[u] = j0 + u < n_splits ? y : -INFINITY;
    }
  };
  // batches past the last split load clamped data with weight 0
  uint4 v0[CB][8];
  float ls0[CB][8];
#pragma unroll
  for (int c = 0; c < CB; c++) {
    load8(8 * c, 8 * l, v0[c]);
    load_lse8(8 * c, ls0[c]);
  }
  __builtin_amdgcn_sched_barrier(0);
  float M = -INFINITY, W = 0.f;  // running max and sum of 2^(lse - M)
  auto fold = [&](const float (&x)[8]) {
    float mb = x[0];
#pragma unroll
    for (int u = 1; u < 8; u++) mb = fmaxf(mb, x[u]);
    if (mb == -INFINITY) return;
    const float Mn = fmaxf(M, mb);
    float s = W * exp2f(M - Mn);  // 0 while M is -inf
#pragma unroll
    for (int u = 0; u < 8; u++) s += exp2f(x[u] - Mn);
    W = s;
    M = Mn;
  };
#pragma unroll
  for (int c = 0; c < CB; c++) fold(ls0[c]);
  for (int j0 = 8 * CB; j0 < n_splits; j0 += 8) {
    float x[8];
    load_lse8(j0, x);
    fold(x);
  }
  uint16_t* ob = out + (size_t)bh * DV;
  if (M == -INFINITY) {
    for (int d = 8 * l; d < DV; d += 8 * kWave) *(uint4*)(ob + d) = uint4{0, 0, 0, 0};
    if (l == 0) lse[bh] = -INFINITY;
    return;
  }
  const float L = M + log2f(W);
  auto accum = [&](const uint4 (&v)[8], const float (&x)[8], float (&a)[8]) {
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const float wj = exp2f(x[u] - L);  // 0 for splits past the end
      const uint32_t y[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        a[2 * e] += wj * __uint_as_float(y[e] << 16);
        a[2 * e + 1] += wj * __uint_as_float(y[e] & 0xFFFF0000u);
      }
    }
  };
  for (int d = 8 * l; d < DV; d += 8 * kWave) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (d == 8 * l) {
#pragma unroll
      for (int c = 0; c < CB; c++) accum(v0[c], ls0[c], a);
    }
    for (int j0 = d == 8 * l ? 8 * CB : 0; j0 < n_splits; j0 += 8) {
      uint4 v[8];
      float x[8];
      load8(j0, d, v);
      load_lse8(j0, x);
      accum(v, x, a);
    }
    uint4 pk;
    pk.x = (uint32_t)f32_to_bf16_rne(a[0]) | ((uint32_t)f32_to_bf16_rne(a[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16_rne(a[2]) | ((uint32_t)f32_to_bf16_rne(a[3]) << 16);
    pk.z = (uint32_t)f32_to_bf16_rne(a[4]) | ((uint32_t)f32_to_bf16_rne(a[5]) << 16);
    pk.w = (uint32_t)f32_to_bf16_rne(a[6]) | ((uint32_t)f32_to_bf16_rne(a[7]) << 16);
    *(uint4*)(ob + d) = pk;
  }
  if (l == 0) lse[bh] = L * kLn2;
}

// The merge for launches with few (request, head) rows, where one wave per
// row would leave most CUs idle (four requests with 32 splits: 512 rows, 128
// workgroups on 256 CUs): one workgroup per row, wave w taking splits
// w, w+4, ...  Each wave keeps its own running max M_w, sum W_w of
// 2^(lse - M_w) and the partials weighted by 2^(lse - M_w) (lane l: dims
// 8l .. 8l+7, all of a wave's loads issued together), then the waves meet
// in LDS: L = M + log2(sum_w W_w 2^(M_w - M)) with M the largest M_w, and
// o = sum_w 2^(M_w - L) acc_w.  DV <= 8 * 64, a multiple of 8; n_splits <=
// 4 * kWideSplitsPerWave.
constexpr int kWideSplitsPerWave = 16;

__global__ __launch_bounds__(256) void k_combine_wide(const uint16_t* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse, int DV,
                                                      int n_splits) {
  __shared__ float sh_m[4], sh_w[4];
  __shared__ __attribute__((aligned(16))) float sh_acc[4][512];
  const int bh = xcd_major(blockIdx.x, gridDim.x);
  const int l = lane_id(), w = wave_id();
  const float* pl = part_lse + (size_t)bh * n_splits;
  const uint16_t* po = part_o + (size_t)bh * n_splits * DV;
  const int dc = min(8 * l, DV - 8);  // lanes past DV load clamped dims, store nothing
  // this wave's splits: w + 4 u (unconditional loads of a clamped split;
  // splits past the end get weight 0)
  uint4 v[kWideSplitsPerWave];
  float x[kWideSplitsPerWave];
#pragma unroll
  for (int u = 0; u < kWideSplitsPerWave; u++) {
    const int j = w + 4 * u;
    const int jc = min(j, n_splits - 1);
    v[u] = *(const uint4*)(po + (size_t)jc * DV + dc);
    const float y = pl[jc];
    x[u] = j < n_splits ? y : -INFINITY;
  }
  float mw = -INFINITY;
#pragma unroll
  for (int u = 0; u < kWideSplitsPerWave; u++) mw = fmaxf(mw, x[u]);
  float ww = 0.f;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (mw != -INFINITY) {
#pragma unroll
    for (int u = 0; u < kWideSplitsPerWave; u++) {
      const float wj = exp2f(x[u] - mw);  // 0 for splits past the end
      ww += wj;
      const uint32_t y[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        a[2 * e] += wj * __uint_as_float(y[e] << 16);
        a[2 * e + 1] += wj * __uint_as_float(y[e] & 0xFFFF0000u);
      }
    }
  }
  if (l == 0) {
    sh_m[w] = mw;
    sh_w[w] = ww;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(sh_m[0], sh_m[1]), fmaxf(sh_m[2], sh_m[3]));
  uint16_t* ob = out + (size_t)bh * DV;
  if (M == -INFINITY) {  // no valid row in any split
    for (int d = 2 * threadIdx.x; d < DV; d += 512) *(uint32_t*)(ob + d) = 0u;
    if (threadIdx.x == 0) lse[bh] = -INFINITY;
    return;
  }
  float W = 0.f;
#pragma unroll
  for (int k = 0; k < 4; k++) W += sh_w[k] * exp2f(sh_m[k] - M);  // 0 for empty waves
  const float L = M + log2f(W);
  const float sc = mw == -INFINITY ? 0.f : exp2f(mw - L);
#pragma unroll
  for (int e = 0; e < 8; e++) sh_acc[w][8 * l + e] = a[e] * sc;
  __syncthreads();
  // thread t: dims 2t, 2t+1
  for (int d = 2 * threadIdx.x; d < DV; d += 512) {
    const float o0 = sh_acc[0][d] + sh_acc[1][d] + sh_acc[2][d] + sh_acc[3][d];
    const float o1 = sh_acc[0][d + 1] + sh_acc[1][d + 1] + sh_acc[2][d + 1] + sh_acc[3][d + 1];
    *(uint32_t*)(ob + d) =
        (uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16);
  }
  if (threadIdx.x == 0) lse[bh] = L * kLn2;
}

// ---------------------------------------------------------------- launchers --

bool attn_uses_mfma(int Hq, int n_kv, int qk_dim, int v_dim, const void* k, const void* v) {
  return n_kv == 1 && k == v && qk_dim == 576 && v_dim == 512 && Hq % 16 == 0;
}

int attn_auto_splits(int B, int Hq, int K, bool mfma) {
  if (!mfma) return 1;
  // one workgroup per CU: aim for about 256 workgroups
  const int groups = (Hq + kHeadsPerWave * kAttnWaves - 1) / (kHeadsPerWave * kAttnWaves);
  int s = (256 + B * groups - 1) / (B * groups);
  const int max_s = (K + kTileR - 1) / kTileR;
  if (s > 32) s = 32;
  if (s > max_s) s = max_s;
  const int min_s = (K + kMaxSplitRows - 1) / kMaxSplitRows;
  if (s < min_s) s = min_s;
  if (s < 1) s = 1;
  return s;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (attn_uses_mfma(a.Hq, a.n_kv, a.qk_dim, a.v_dim, a.k, a.v)) {
    const int rps = ((a.K + a.n_splits - 1) / a.n_splits + kTileR - 1) / kTileR * kTileR;
    if (rps > kMaxSplitRows) return hipErrorInvalidValue;
    const int hpw = kHeadsPerWave * kAttnWaves;
    dim3 grid(a.n_splits, (a.Hq + hpw - 1) / hpw, a.B);
    if (a.gather.src) {
      // the gathering form writes the hot buffer: its grid must cover each
      // split once (one head group)
      if (grid.y != 1) return hipErrorInvalidValue;
      hipLaunchKernelGGL((k_attn_mfma<576, 512, kAttnBufs, true>), grid, dim3(64 * kAttnWaves),
                         0, st, a.q, a.k, a.rows, a.out, a.lse, a.part_o, a.part_lse, a.Hq, a.K,
                         a.rows_per_req, a.row_stride, a.scale * kLog2e, a.n_splits, rps,
                         a.gather);
    } else {
      hipLaunchKernelGGL((k_attn_mfma<576, 512, kAttnBufs, false>), grid, dim3(64 * kAttnWaves),
                         0, st, a.q, a.k, a.rows, a.out, a.lse, a.part_o, a.part_lse, a.Hq, a.K,
                         a.rows_per_req, a.row_stride, a.scale * kLog2e, a.n_splits, rps,
                         a.gather);
    }
  } else {
    if (a.qk_dim % 8 != 0 || a.v_dim % 8 != 0 || a.qk_dim > kValuMaxDim ||
        a.v_dim > kValuMaxDim || a.K > kValuMaxRows)
      return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_attn_valu<8>, dim3(a.Hq, a.B), dim3(256), 0, st, a.q, a.k, a.v, a.rows,
                       a.out, a.lse, a.Hq, a.n_kv, a.qk_dim, a.v_dim, a.K, a.rows_per_req,
                       a.row_stride, a.head_stride, a.scale);
  }
  return hipGetLastError();
}

// The one-workgroup-per-row merge when one wave per row would fill fewer
// than 256 workgroups (about one per CU) and each wave still gets at least
// two splits.
bool combine_uses_wide(int BH, int DV, int n_splits) {
  return (BH + 3) / 4 < 256 && n_splits >= 8 && n_splits <= 4 * kWideSplitsPerWave &&
         DV <= 512;
}

hipError_t launch_combine(const AttnArgs& a, hipStream_t st) {
  if (a.v_dim % 8 != 0) return hipErrorInvalidValue;
  const int BH = a.B * a.Hq;
  if (combine_uses_wide(BH, a.v_dim, a.n_splits)) {
    hipLaunchKernelGGL(k_combine_wide, dim3(BH), dim3(256), 0, st, a.part_o, a.part_lse, a.out,
                       a.lse, a.v_dim, a.n_splits);
    return hipGetLastError();
  }
  if (a.n_splits > 8)
    hipLaunchKernelGGL(k_combine<4>, dim3((BH + 3) / 4), dim3(256), 0, st, a.part_o, a.part_lse,
                       a.out, a.lse, BH, a.v_dim, a.n_splits);
  else
    hipLaunchKernelGGL(k_combine<1>, dim3((BH + 3) / 4), dim3(256), 0, st, a.part_o, a.part_lse,
                       a.out, a.lse, BH, a.v_dim, a.n_splits);
  return hipGetLastError();
}

}  // namespace ls
