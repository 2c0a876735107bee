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

// Workgroups are dispatched to the eight XCDs in turn (id mod 8), and each
// XCD has its own L2.  xcd_major renumbers a grid of n workgroups so that
// consecutive new ids run on one XCD: workgroups that share data (the splits
// of one request, say) then share that XCD's L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_major(int id, int n) {
  const int x = id & 7, j = id >> 3, per = n >> 3, rem = n & 7;
  return x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

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

// Lane swaps of gfx950 (VALU, no LDS round trip).  permlane32_swap(X, Y)
// exchanges the upper 32 lanes of X with the lower 32 lanes of Y;
// permlane16_swap(X, Y) exchanges the odd 16-lane rows of X with the even
// rows of Y.  The 64-bit forms move each 32-bit word the same way.
__device__ __forceinline__ void swap32(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}
__device__ __forceinline__ void swap32(uint64_t& x, uint64_t& y) {
  uint32_t xl = (uint32_t)x, xh = (uint32_t)(x >> 32), yl = (uint32_t)y, yh = (uint32_t)(y >> 32);
  swap32(xl, yl);
  swap32(xh, yh);
  x = ((uint64_t)xh << 32) | xl;
  y = ((uint64_t)yh << 32) | yl;
}
__device__ __forceinline__ void swap16(uint64_t& x, uint64_t& y) {
  uint32_t xl = (uint32_t)x, xh = (uint32_t)(x >> 32), yl = (uint32_t)y, yh = (uint32_t)(y >> 32);
  swap16(xl, yl);
  swap16(xh, yh);
  x = ((uint64_t)xh << 32) | xl;
  y = ((uint64_t)yh << 32) | yl;
}

// Reduce-scatter over the four 16-lane groups g = lane/16 (sums modulo
// 2^bits of U): on entry p_tt is this lane's partial for (tile tt, lane%16);
// on exit the result is the full sum for tile g, lane%16.  Swapping (p0, p2)
// leaves every lane with the partials of lanes l and l^32 for tile 0 (lanes
// < 32) or tile 2 (lanes >= 32), and (p1, p3) likewise for tiles 1 / 3; the
// 16-lane swap of those sums then pairs groups g and g^1.
template <class U>
__device__ __forceinline__ U reduce_scatter4(U p0, U p1, U p2, U p3) {
  swap32(p0, p2);
  swap32(p1, p3);
  U k0 = p0 + p2, k1 = p1 + p3;
  swap16(k0, k1);
  return k0 + k1;
}

// x of lanes l and l^32: the pair (lower lane's, upper lane's) in every lane.
__device__ __forceinline__ void pair32(float x, float& lo, float& hi) {
  uint32_t a = __float_as_uint(x), b = a;
  swap32(a, b);
  lo = __uint_as_float(a);
  hi = __uint_as_float(b);
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
typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}

// One 1 KiB global -> LDS copy (global_load_lds_dwordx4): lane i's 16 bytes
// at src land at LDS byte lds_base + 16 i (lds_base wave-uniform).  Written
// out so that the compiler neither reorders LDS accesses across it nor
// counts it: the caller waits for it with an explicit vmcnt.  It has no VGPR
// destination, so nothing it writes can be reused while it is in flight.
// m0 is a reserved register that the compiler never holds a value in across
// other code on gfx950 (it sets m0 right before the few instructions that read
// it), so the clobber below only documents the write; clang warns that it
// names a reserved register, which is expected here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// 24-bit signed multiply-add, c + a * b modulo 2^32 (one v_mad_i32_i24; the
// compiler would otherwise split the chain into multiplies and 3-way adds).
__device__ __forceinline__ uint32_t mad_i24(int32_t a, int32_t b, uint32_t c) {
  uint32_t d;
  asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// Raw buffer resource over [p, p + bytes) (stride 0, gfx9 dword-3 format
// word): the hardware range check drops stores at offsets beyond `bytes` and
// returns 0 for such loads, so edge lanes need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ int clamp_ctx(const int32_t* ctx_len, int b, int max_ctx) {
  int n = ctx_len[b];
  return n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
}

}  // namespace ls
