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
// k_combine    -- merges the per-split partials (normalised o, log2-lse).
#include "ls_device.h"
#include "ls_launch.h"

namespace ls {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- MFMA path --
//
// Workgroup = NW waves x 16 query heads, one request, one split of the row
// list.  Rows are staged 32 at a time in LDS, row-major (padded stride).
// Q stays in VGPRs as the B operand of S^T = K Q^T (lane: head n = lane%16,
// dims 8*(lane/16) .. +8 of each 32-dim step); the K tile gives the A
// operand (16 rows x 8 dims per lane).  The S^T accumulator leaves every
// lane with 8 scores of its own head, rows 4g..4g+3 and 16+4g..16+4g+3
// (g = lane/16); converted to bf16 they are the B operand of O^T = V^T P^T
// with that row order.  The matching A operand -- 8 rows of one V column --
// comes straight from the row-major tile through the gfx950 LDS transpose
// read (ds_read_b64_tr_b16): within each 16-lane group, lane j points at
// row base + j/4, columns 4*(j%4) .. +3, and lane i receives column i of
// those 4 rows; two such reads (row bases 4g and 16+4g) give the 8 rows.
// O^T accumulates 16 dims x 16 heads per MFMA, so every lane owns one head's
// outputs and the online-softmax rescale is lane-local.
constexpr int kTileR = 32;

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i16 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
}

template <int DQK, int DV, int NW>
__global__ __launch_bounds__(NW * 64, 2) void k_attn_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ rows, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse, int Hq, int K,
    int64_t rows_per_req, int64_t row_stride, float scale_log2, int n_splits,
    int rows_per_split) {
  constexpr int NT = NW * 64;
  constexpr int KS = DQK + 8;     // LDS row stride of the tile (bf16 elements)
  constexpr int QK_STEPS = DQK / 32;
  constexpr int DT = DV / 16;
  constexpr int CH = DQK / 8;     // 16-byte chunks per row
  constexpr int CPT = NT / kTileR;              // chunk lanes per row
  constexpr int LPT = (CH + CPT - 1) / CPT;     // chunk loads per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kTileR * KS];

  const int split = blockIdx.x, b = blockIdx.z;
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const int h = blockIdx.y * (16 * NW) + wave_id() * 16 + n;
  const bool h_ok = h < Hq;

  v8bf qB[QK_STEPS];
  {
    const uint16_t* qh = q + ((size_t)b * Hq + (h_ok ? h : 0)) * DQK;
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ks++) {
      v8u16 v = h_ok ? *(const v8u16*)(qh + 32 * ks + 8 * g) : v8u16{0, 0, 0, 0, 0, 0, 0, 0};
      qB[ks] = __builtin_bit_cast(v8bf, v);
    }
  }
  v4f oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) oacc[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int i_begin = split * rows_per_split;
  const int i_end = min(i_begin + rows_per_split, K);
  const int32_t* rb = rows + (size_t)b * K;
  const uint16_t* kvb = kv + (size_t)b * rows_per_req * row_stride;
  // this thread stages row lr of every tile, chunks lc, lc + CPT, ...
  const int lr = threadIdx.x % kTileR, lc = threadIdx.x / kTileR;

  for (int tile0 = i_begin; tile0 < i_end; tile0 += kTileR) {
    const int i = tile0 + lr;
    const int32_t rid = (i < i_end) ? rb[i] : -1;
    // every wave holds rows 0..31 in lanes 0..31: the tile's validity mask
    const uint32_t vmask = (uint32_t)__ballot(rid >= 0);
    const uint16_t* src = kvb + (size_t)(rid >= 0 ? rid : 0) * row_stride;
    // two batches of chunk loads keep the staging registers small: the first
    // is in flight across the barrier, the second right after it
    constexpr int LA = (LPT + 1) / 2;
    uint4 v[LA];
#pragma unroll
    for (int j = 0; j < LA; j++) {
      const int c = lc + CPT * j;
      v[j] = (c < CH && rid >= 0) ? *(const uint4*)(src + 8 * c) : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();  // the previous tile is no longer read
#pragma unroll
    for (int j = 0; j < LA; j++) {
      const int c = lc + CPT * j;
      if (c < CH) *(uint4*)&Ks[lr * KS + 8 * c] = v[j];
    }
#pragma unroll
    for (int j = LA; j < LPT; j++) {
      const int c = lc + CPT * j;
      v[j - LA] = (c < CH && rid >= 0) ? *(const uint4*)(src + 8 * c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = LA; j < LPT; j++) {
      const int c = lc + CPT * j;
      if (c < CH) *(uint4*)&Ks[lr * KS + 8 * c] = v[j - LA];
    }
    __syncthreads();

    // S^T = K Q^T for rows 0..15 and 16..31
    v4f sacc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ks++) {
#pragma unroll
      for (int rt = 0; rt < 2; rt++) {
        v8u16 a = *(const v8u16*)&Ks[(16 * rt + n) * KS + 32 * ks + 8 * g];
        sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), qB[ks],
                                                            sacc[rt], 0, 0, 0);
      }
    }
    float s[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int r = (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4);
      const float sv = (e < 4) ? sacc[0][e] : sacc[1][e - 4];
      s[e] = ((vmask >> r) & 1u) ? sv * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, s[e]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    // Branch-free when no row is valid yet (m_new = -inf): alpha = 0 on a
    // zero accumulator and every p = 0.  MFMAs stay outside divergent code.
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_ref);
    float psum = 0.f;
    uint16_t pb[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const float p = exp2f(s[e] - m_ref);
      psum += p;
      pb[e] = f32_to_bf16_rne(p);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;  // stays -inf until a valid row appears
    v8u16 pv = {pb[0], pb[1], pb[2], pb[3], pb[4], pb[5], pb[6], pb[7]};
    const v8bf pB = __builtin_bit_cast(v8bf, pv);
    // transpose-read addresses: lane j of the group -> row base + j/4, cols 4*(j%4)
    const uint16_t* tr0 = &Ks[(4 * g + (n >> 2)) * KS + 4 * (n & 3)];
    const uint16_t* tr1 = tr0 + 16 * KS;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
      oacc[dt] *= alpha;
      const v4i16 a0 = lds_read_tr16(tr0 + 16 * dt);
      const v4i16 a1 = lds_read_tr16(tr1 + 16 * dt);
      const v8u16 a = {(uint16_t)a0[0], (uint16_t)a0[1], (uint16_t)a0[2], (uint16_t)a0[3],
                       (uint16_t)a1[0], (uint16_t)a1[1], (uint16_t)a1[2], (uint16_t)a1[3]};
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), pB,
                                                          oacc[dt], 0, 0, 0);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  if (!h_ok) return;
  const bool any = l_tot > 0.f;
  const float inv = any ? 1.f / l_tot : 0.f;
  const float lse2 = any ? m_run + log2f(l_tot) : -INFINITY;
  if (n_splits == 1) {
    uint16_t* ob = out + ((size_t)b * Hq + h) * DV;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
      const int d = 16 * dt + 4 * g;
      uint2 v;
      v.x = (uint32_t)f32_to_bf16_rne(oacc[dt][0] * inv) |
            ((uint32_t)f32_to_bf16_rne(oacc[dt][1] * inv) << 16);
      v.y = (uint32_t)f32_to_bf16_rne(oacc[dt][2] * inv) |
            ((uint32_t)f32_to_bf16_rne(oacc[dt][3] * inv) << 16);
      *(uint2*)(ob + d) = v;
    }
    if (g == 0) lse[(size_t)b * Hq + h] = any ? lse2 * kLn2 : -INFINITY;
  } else {
    const size_t ps = ((size_t)b * Hq + h) * n_splits + split;
    float* po = part_o + ps * DV;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
      const int d = 16 * dt + 4 * g;
      *(float4*)(po + d) = make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv,
                                       oacc[dt][2] * inv, oacc[dt][3] * inv);
    }
    if (g == 0) part_lse[ps] = lse2;
  }
}

// ---------------------------------------------------------------- VALU path --
// One workgroup per (query head, request): scores in LDS, block softmax, then
// the weighted sum of V rows with threads over (row group, dim).
constexpr int kValuMaxRows = 8192;
constexpr int kValuMaxDim = 1024;

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

__global__ __launch_bounds__(256) void k_attn_valu(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kbase,
    const uint16_t* __restrict__ vbase, const int32_t* __restrict__ rows,
    uint16_t* __restrict__ out, float* __restrict__ lse, int Hq, int n_kv, int dqk, int dv,
    int K, int64_t rows_per_req, int64_t row_stride, int64_t head_stride, float scale) {
  __shared__ float qs[kValuMaxDim];
  __shared__ float sc[kValuMaxRows];
  __shared__ float red[4];
  __shared__ float acc_sh[256];
  const int h = blockIdx.x, b = blockIdx.y;
  const int kvh = h / (Hq / n_kv);
  const int tid = threadIdx.x, l = lane_id(), wv = wave_id();
  const uint16_t* qh = q + ((size_t)b * Hq + h) * dqk;
  for (int d = tid; d < dqk; d += 256) qs[d] = bf16_to_f32(qh[d]);
  __syncthreads();
  const int32_t* rb = rows + (size_t)b * K;
  const size_t req_off = (size_t)b * rows_per_req * row_stride + (size_t)kvh * head_stride;
  for (int i = wv; i < K; i += 4) {
    const int32_t r = rb[i];
    float dot = 0.f;
    if (r >= 0) {
      const uint16_t* kr = kbase + req_off + (size_t)r * row_stride;
      for (int d = l; d < dqk; d += 64) dot += qs[d] * bf16_to_f32(kr[d]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o, kWave);
    if (l == 0) sc[i] = (r >= 0) ? dot * scale : -INFINITY;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int i = tid; i < K; i += 256) m = fmaxf(m, sc[i]);
  m = block_reduce_max(m, red);
  float lsum = 0.f;
  if (m != -INFINITY) {
    for (int i = tid; i < K; i += 256) {
      const float p = (sc[i] == -INFINITY) ? 0.f : expf(sc[i] - m);
      sc[i] = p;
      lsum += p;
    }
  }
  lsum = block_reduce_sum(lsum, red);
  __syncthreads();
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* ob = out + ((size_t)b * Hq + h) * dv;
  // threads = (row group rg, dim d); dims in chunks of at most 256
  for (int d0 = 0; d0 < dv; d0 += 256) {
    const int nd = min(256, dv - d0);
    const int groups = 256 / nd;
    const int d = d0 + tid % nd, rg = tid / nd;
    float acc = 0.f;
    if (rg < groups && m != -INFINITY) {
      for (int i = rg; i < K; i += groups) {
        const int32_t r = rb[i];
        if (r >= 0) acc += sc[i] * bf16_to_f32(vbase[req_off + (size_t)r * row_stride + d]);
      }
    }
    acc_sh[tid] = (rg < groups) ? acc : 0.f;
    __syncthreads();
    if (tid < nd) {
      float tot = 0.f;
      for (int k = 0; k < groups; k++) tot += acc_sh[k * nd + tid];
      ob[d0 + tid] = f32_to_bf16_rne(tot * inv);
    }
    __syncthreads();
  }
  if (tid == 0) lse[(size_t)b * Hq + h] = (lsum > 0.f) ? m + logf(lsum) : -INFINITY;
}

// ------------------------------------------------------------------ combine --
// out = sum_j o_j 2^(lse_j - L) with L = log2 sum_j 2^lse_j; lse = L ln 2.
__global__ __launch_bounds__(128) void k_combine(const float* __restrict__ part_o,
                                                 const float* __restrict__ part_lse,
                                                 uint16_t* __restrict__ out,
                                                 float* __restrict__ lse, int DV,
                                                 int n_splits) {
  const size_t bh = blockIdx.x;
  const float* pl = part_lse + bh * n_splits;
  float M = -INFINITY;
  for (int j = 0; j < n_splits; j++) M = fmaxf(M, pl[j]);
  uint16_t* ob = out + bh * DV;
  if (M == -INFINITY) {
    for (int d = threadIdx.x; d < DV; d += 128) ob[d] = 0;
    if (threadIdx.x == 0) lse[bh] = -INFINITY;
    return;
  }
  float W = 0.f;
  for (int j = 0; j < n_splits; j++) W += exp2f(pl[j] - M);
  const float L = M + log2f(W);
  const float* po = part_o + bh * n_splits * DV;
  for (int d = threadIdx.x * 4; d < DV; d += 128 * 4) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < n_splits; j++) {
      const float wj = exp2f(pl[j] - L);
      if (wj == 0.f) continue;
      const float4 v = *(const float4*)(po + (size_t)j * DV + d);
      a.x += wj * v.x;
      a.y += wj * v.y;
      a.z += wj * v.z;
      a.w += wj * v.w;
    }
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16_rne(a.x) | ((uint32_t)f32_to_bf16_rne(a.y) << 16);
    pk.y = (uint32_t)f32_to_bf16_rne(a.z) | ((uint32_t)f32_to_bf16_rne(a.w) << 16);
    *(uint2*)(ob + d) = pk;
  }
  if (threadIdx.x == 0) lse[bh] = L * kLn2;
}

// ---------------------------------------------------------------- launchers --

bool attn_uses_mfma(int Hq, int n_kv, int qk_dim, int v_dim, const void* k, const void* v) {
  return n_kv == 1 && k == v && qk_dim == 576 && v_dim == 512 && Hq % 16 == 0;
}

int attn_auto_splits(int B, int Hq, int K, bool mfma) {
  if (!mfma) return 1;
  const int groups = (Hq + 63) / 64;
  int s = (512 + B * groups - 1) / (B * groups);
  const int max_s = (K + kTileR - 1) / kTileR;
  if (s > 16) s = 16;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return s;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (attn_uses_mfma(a.Hq, a.n_kv, a.qk_dim, a.v_dim, a.k, a.v)) {
    const int rps = ((a.K + a.n_splits - 1) / a.n_splits + kTileR - 1) / kTileR * kTileR;
    dim3 grid(a.n_splits, (a.Hq + 63) / 64, a.B);
    hipLaunchKernelGGL((k_attn_mfma<576, 512, 4>), grid, dim3(256), 0, st, a.q, a.k, a.rows,
                       a.out, a.lse, a.part_o, a.part_lse, a.Hq, a.K, a.rows_per_req,
                       a.row_stride, a.scale * kLog2e, a.n_splits, rps);
  } else {
    hipLaunchKernelGGL(k_attn_valu, dim3(a.Hq, a.B), dim3(256), 0, st, a.q, a.k, a.v, a.rows,
                       a.out, a.lse, a.Hq, a.n_kv, a.qk_dim, a.v_dim, a.K, a.rows_per_req,
                       a.row_stride, a.head_stride, a.scale);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const AttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_combine, dim3(a.B * a.Hq), dim3(128), 0, st, a.part_o, a.part_lse, a.out,
                     a.lse, a.v_dim, a.n_splits);
  return hipGetLastError();
}

}  // namespace ls
