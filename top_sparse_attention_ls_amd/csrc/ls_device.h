// Device helpers shared by the gfx950 kernels of libls.so: wave and block
// scans, the block-cooperative radix threshold search used by every
// selection, MFMA operand types and bf16 conversion.
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

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t t = __shfl_up(v, o, kWave);
    if (lane_id() >= o) v += t;
  }
  return v;
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
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
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

// Result of a threshold search: an entry (key u, position p) is kept iff
//   mode 0:  u >= key
//   mode 1:  u > key, or u == key and p <= pos.
struct Threshold {
  uint64_t key;
  uint32_t pos;
  int mode;
};

__device__ __forceinline__ bool keep(const Threshold& t, uint64_t u, uint32_t p) {
  return t.mode == 0 ? (u >= t.key) : (u > t.key || (u == t.key && p <= t.pos));
}

struct SelectShared {
  uint32_t hist[256];
  uint64_t red[2][16];
  uint32_t beta, before, cnt;
};

// Block reduction of (min, max) of unsigned 64-bit keys.  NT threads.
template <int NT>
__device__ __forceinline__ void block_minmax(uint64_t& mn, uint64_t& mx, SelectShared& sh) {
  mn = wave_min_u64(mn);
  mx = wave_max_u64(mx);
  if (lane_id() == 0) {
    sh.red[0][wave_id()] = mn;
    sh.red[1][wave_id()] = mx;
  }
  __syncthreads();
  mn = sh.red[0][0];
  mx = sh.red[1][0];
#pragma unroll
  for (int i = 1; i < NT / kWave; i++) {
    mn = sh.red[0][i] < mn ? sh.red[0][i] : mn;
    mx = sh.red[1][i] > mx ? sh.red[1][i] : mx;
  }
  __syncthreads();
}

// Wave 0 finds the bin where the running count crosses `need`, counting
// from the top bin down (from_top) or from bin 0 up.  Writes beta, the count
// strictly before it in that direction, and the bin's own count.
__device__ __forceinline__ void find_crossing(SelectShared& sh, uint32_t need, bool from_top) {
  if (wave_id() != 0) return;
  const int l = lane_id();
  uint32_t c0 = sh.hist[4 * l], c1 = sh.hist[4 * l + 1], c2 = sh.hist[4 * l + 2],
           c3 = sh.hist[4 * l + 3];
  uint32_t s = c0 + c1 + c2 + c3;
  uint32_t excl = from_top ? wave_incl_suffix(s) - s : wave_incl_scan(s) - s;
  if (excl < need && need <= excl + s) {
    uint32_t c[4] = {c0, c1, c2, c3};
    uint32_t run = excl;
    for (int k = 0; k < 4; k++) {
      int kk = from_top ? 3 - k : k;
      if (run + c[kk] >= need) {
        sh.beta = 4 * l + kk;
        sh.before = run;
        sh.cnt = c[kk];
        break;
      }
      run += c[kk];
    }
  }
}

// Block-cooperative threshold search over n entries (key, position), keys
// unsigned, positions unique.  Finds the threshold that keeps exactly `need`
// entries (1 <= need < n) under the order key descending, position
// ascending, by narrowing 8-bit digits of the key from the first bit where
// the entries differ, then digits of the position among entries tied at the
// cut key.  get(i, u, p) loads entry i.  NT threads; every thread returns
// the same threshold.
template <int NT, class Get>
__device__ Threshold block_threshold(const Get& get, int n, uint32_t need, SelectShared& sh) {
  const int tid = threadIdx.x;
  uint64_t mn = ~0ull, mx = 0;
  for (int i = tid; i < n; i += NT) {
    uint64_t u;
    uint32_t p;
    get(i, u, p);
    mn = u < mn ? u : mn;
    mx = u > mx ? u : mx;
  }
  block_minmax<NT>(mn, mx, sh);

  // ---- key digits, from the top
  int nb = (mn == mx) ? 0 : 64 - __clzll(mx ^ mn);
  uint64_t prefix = (nb >= 64) ? 0ull : ((mx >> nb) << nb);
  while (nb > 0) {
    const int d = nb < 8 ? nb : 8;
    const int shft = nb - d;
    const uint64_t dmask = (1ull << d) - 1ull;
    for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      uint64_t u;
      uint32_t p;
      get(i, u, p);
      bool in = (nb >= 64) || ((u >> nb) == (prefix >> nb));
      if (in) atomicAdd(&sh.hist[(uint32_t)((u >> shft) & dmask)], 1u);
    }
    __syncthreads();
    find_crossing(sh, need, true);
    __syncthreads();
    const uint32_t beta = sh.beta, before = sh.before, cnt = sh.cnt;
    __syncthreads();
    need -= before;
    prefix |= (uint64_t)beta << shft;
    nb = shft;
    if (cnt == need) return Threshold{prefix, 0u, 0};
  }

  // ---- every remaining candidate has key == prefix: smallest positions win
  const uint64_t cut = prefix;
  uint64_t pmn = ~0ull, pmx = 0;
  for (int i = tid; i < n; i += NT) {
    uint64_t u;
    uint32_t p;
    get(i, u, p);
    if (u == cut) {
      pmn = p < pmn ? p : pmn;
      pmx = p > pmx ? p : pmx;
    }
  }
  block_minmax<NT>(pmn, pmx, sh);
  int pb = (pmn == pmx) ? 0 : 64 - __clzll(pmx ^ pmn);
  uint64_t pprefix = (pb >= 64) ? 0ull : ((pmn >> pb) << pb);
  while (pb > 0) {
    const int d = pb < 8 ? pb : 8;
    const int shft = pb - d;
    const uint64_t dmask = (1ull << d) - 1ull;
    for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      uint64_t u;
      uint32_t p;
      get(i, u, p);
      if (u == cut && ((uint64_t)p >> pb) == (pprefix >> pb))
        atomicAdd(&sh.hist[(uint32_t)(((uint64_t)p >> shft) & dmask)], 1u);
    }
    __syncthreads();
    find_crossing(sh, need, false);
    __syncthreads();
    const uint32_t beta = sh.beta, before = sh.before, cnt = sh.cnt;
    __syncthreads();
    need -= before;
    pprefix |= (uint64_t)beta << shft;
    pb = shft;
    if (cnt == need) return Threshold{cut, (uint32_t)(pprefix + ((1ull << shft) - 1ull)), 1};
  }
  return Threshold{cut, (uint32_t)pprefix, 1};
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
