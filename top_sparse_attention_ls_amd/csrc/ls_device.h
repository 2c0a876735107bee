// Device helpers shared by the gfx950 kernels of libls.so: wave and block
// scans, order-preserving keys, MFMA operand types and bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ls {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// Lanes below this one whose bit is set in mask (the wave's own rank).
__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// DPP lane move within the wave; lanes without a source (or outside
// row_mask) contribute 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the wave on DPP moves (row_shr 1/2/4/8 within
// each 16-lane row, then row_bcast 15 and 31 across rows).  Every lane of
// the wave must be active.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_or_zero<0x111, 0xF>(v);
  v += dpp_or_zero<0x112, 0xF>(v);
  v += dpp_or_zero<0x114, 0xF>(v);
  v += dpp_or_zero<0x118, 0xF>(v);
  v += dpp_or_zero<0x142, 0xA>(v);
  v += dpp_or_zero<0x143, 0xC>(v);
  return v;
}

// Value of lane src (wave-uniform) in every lane.
__device__ __forceinline__ uint32_t wave_read(uint32_t v, int src) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, src);
}

// Sum over this lane and every higher lane.
__device__ __forceinline__ uint32_t wave_incl_suffix(uint32_t v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t t = __shfl_down(v, o, kWave);
    if (lane_id() + o < kWave) v += t;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return wave_read(wave_incl_scan(v), kWave - 1);
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t t = __shfl_xor(v, o, kWave);
    v = t < v ? t : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t t = __shfl_xor(v, o, kWave);
    v = t > v ? t : v;
  }
  return v;
}

// Exclusive prefix sum over the NT threads of a block; *total gets the sum.
// sh must hold NT / 64 words of LDS.  Contains two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
  uint32_t inc = wave_incl_scan(v);
  const int w = wave_id();
  if (lane_id() == kWave - 1) sh[w] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; i++) {
    uint32_t s = sh[i];
    base += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// ----------------------------------------------------------------------------
// Order-preserving maps of signed scores onto unsigned keys.
__device__ __forceinline__ uint64_t key_of_i32(int32_t x) {
  return (uint64_t)((uint32_t)x ^ 0x80000000u);
}
__device__ __forceinline__ uint64_t key_of_i64(int64_t x) {
  return (uint64_t)x ^ 0x8000000000000000ull;
}

// ----------------------------------------------------------------------------
// float -> bfloat16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Valid token count of request b, clamped to [0, max_ctx].
__device__ __forceinline__ int clamp_ctx(const int32_t* ctx_len, int b, int max_ctx) {
  int n = ctx_len[b];
  return n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
}

}  // namespace ls
