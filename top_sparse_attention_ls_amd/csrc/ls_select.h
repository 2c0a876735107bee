// Exact threshold searches of the selections: which entries (key, position)
// are kept when exactly `need` of them survive under the order key
// descending, position ascending.  Two forms: one wave on its own (no
// workgroup barriers; for the short tie lists left after a histogram pass)
// and the whole workgroup (for long lists).
#pragma once

#include "ls_device.h"

namespace ls {

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
  __attribute__((aligned(16))) uint32_t hist[256];
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

// hist[bin] += 1 for every active lane with `on`.  The lanes that share the
// bin of the wave's first such lane add with one atomic between them, so a
// run of equal keys costs one LDS atomic per wave rather than one per lane
// (same-address atomics serialise); the other lanes add their own.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool on) {
  const uint64_t act = __ballot(on);
  if (act == 0) return;
  const int first = __ffsll((unsigned long long)act) - 1;
  const uint32_t b0 = wave_read(bin, first);
  const uint64_t same = __ballot(on && bin == b0);
  if (on) {
    if (bin != b0)
      atomicAdd(&hist[bin], 1u);
    else if ((int)lane_id() == first)
      atomicAdd(&hist[b0], (uint32_t)__popcll(same));
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
    for (int i0 = 0; i0 < n; i0 += NT) {  // whole waves: hist_add is per wave
      const int i = i0 + tid;
      uint64_t u;
      uint32_t p;
      get(min(i, n - 1), u, p);
      const bool in = i < n && ((nb >= 64) || ((u >> nb) == (prefix >> nb)));
      hist_add(sh.hist, (uint32_t)((u >> shft) & dmask), in);
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
    for (int i0 = 0; i0 < n; i0 += NT) {  // whole waves: hist_add is per wave
      const int i = i0 + tid;
      uint64_t u;
      uint32_t p;
      get(min(i, n - 1), u, p);
      // (runs of consecutive positions -- bursts of equal scores -- share a bin)
      hist_add(sh.hist, (uint32_t)(((uint64_t)p >> shft) & dmask),
               i < n && u == cut && ((uint64_t)p >> pb) == (pprefix >> pb));
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
// The same search done by one wave alone, for lists whose keys are known to
// lie in [key_lo, key_hi] (the range of the histogram bucket they came from)
// and whose positions are below 2^pos_bits: no reductions are needed to find
// the first bit where entries can differ.  hist is 256 words (16-byte
// aligned) of LDS that only this wave touches.  Every lane returns the
// threshold.  All 64 lanes must be active.
// Bits needed for positions below n (n >= 1).
__device__ __forceinline__ int pos_bits_below(int n) {
  return n <= 1 ? 0 : 32 - __clz(n - 1);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Narrows one 8-bit digit: counts the entries that `entry` accepts into
// hist by digit and finds the bin where the count (from the top bin down, or
// from bin 0 up) reaches need.  Returns the bin, the count before it and the
// bin's own count.
template <class Entry>
__device__ __forceinline__ void wave_digit(const Entry& entry, int n, uint32_t* hist,
                                           bool from_top, uint32_t need, uint32_t* beta,
                                           uint32_t* before, uint32_t* cnt) {
  const int l = lane_id();
  *(uint4*)&hist[4 * l] = make_uint4(0u, 0u, 0u, 0u);
  wave_lds_sync();
  for (int i0 = l; i0 < n; i0 += 4 * kWave) {
    uint32_t d[4];
    bool m[4];
    // entries read unconditionally (index clamped, n >= 1), so the four
    // reads are in flight together instead of one branch and wait each
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int i = i0 + j * kWave;
      d[j] = 0;
      const bool ok = entry(min(i, n - 1), d[j]);
      m[j] = i < n && ok;
    }
#pragma unroll
    for (int j = 0; j < 4; j++)
      if (m[j]) atomicAdd(&hist[d[j]], 1u);
  }
  wave_lds_sync();
  // lane l owns four bins; counted from the top, lane 0 owns bins 255..252
  const int g = from_top ? kWave - 1 - l : l;
  const uint4 h = *(const uint4*)&hist[4 * g];
  uint32_t c[4];
  if (from_top) {
    c[0] = h.w; c[1] = h.z; c[2] = h.y; c[3] = h.x;
  } else {
    c[0] = h.x; c[1] = h.y; c[2] = h.z; c[3] = h.w;
  }
  const uint32_t s = c[0] + c[1] + c[2] + c[3];
  const uint32_t incl = wave_incl_scan(s);
  const uint32_t excl = incl - s;
  const bool hit = excl < need && need <= incl;
  uint32_t bb = 0, bf = 0, bc = 0, run = excl;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    if (run < need && run + c[k] >= need) {
      bb = from_top ? 4 * g + 3 - k : 4 * g + k;
      bf = run;
      bc = c[k];
    }
    run += c[k];
  }
  const int src = __ffsll((unsigned long long)__ballot(hit)) - 1;
  *beta = wave_read(bb, src);
  *before = wave_read(bf, src);
  *cnt = wave_read(bc, src);
  wave_lds_sync();
}

// LDS scratch of a tie search: the entries that survive the first key digit,
// when few enough, so that the remaining digits run over a short list.
constexpr int kThrScratch = 256;
struct ThresholdScratch {
  uint64_t key[kThrScratch];
  uint32_t pos[kThrScratch];
  uint32_t fill;
};

template <class Get>
__device__ Threshold wave_threshold(const Get& get, int n, uint32_t need, uint32_t* hist,
                                    uint64_t key_lo, uint64_t key_hi, int pos_bits) {
  int nb = (key_lo == key_hi) ? 0 : 64 - __clzll(key_lo ^ key_hi);
  uint64_t prefix = (nb >= 64) ? 0ull : ((key_hi >> nb) << nb);
  while (nb > 0) {
    const int d = nb < 8 ? nb : 8;
    const int shft = nb - d;
    const uint64_t dmask = (1ull << d) - 1ull;
    auto entry = [&](int i, uint32_t& dg) {
      uint64_t u;
      uint32_t p;
      get(i, u, p);
      dg = (uint32_t)((u >> shft) & dmask);
      return (nb >= 64) || ((u >> nb) == (prefix >> nb));
    };
    uint32_t beta, before, cnt;
    wave_digit(entry, n, hist, true, need, &beta, &before, &cnt);
    need -= before;
    prefix |= (uint64_t)beta << shft;
    nb = shft;
    if (cnt == need) return Threshold{prefix, 0u, 0};
  }
  // every remaining entry has key == prefix: smallest positions win
  const uint64_t cut = prefix;
  int pb = pos_bits;
  uint64_t pprefix = 0;
  while (pb > 0) {
    const int d = pb < 8 ? pb : 8;
    const int shft = pb - d;
    const uint64_t dmask = (1ull << d) - 1ull;
    auto entry = [&](int i, uint32_t& dg) {
      uint64_t u;
      uint32_t p;
      get(i, u, p);
      dg = (uint32_t)(((uint64_t)p >> shft) & dmask);
      return u == cut && ((uint64_t)p >> pb) == (pprefix >> pb);
    };
    uint32_t beta, before, cnt;
    wave_digit(entry, n, hist, false, need, &beta, &before, &cnt);
    need -= before;
    pprefix |= (uint64_t)beta << shft;
    pb = shft;
    if (cnt == need) return Threshold{cut, (uint32_t)(pprefix + ((1ull << shft) - 1ull)), 1};
  }
  return Threshold{cut, (uint32_t)pprefix, 1};
}

// ----------------------------------------------------------------------------
// The tie search of the selections: the exact threshold over a list whose
// keys lie in [key_lo, key_hi] (a histogram bucket's range).  The first key
// digit -- the only step that touches every entry -- is counted by the whole
// workgroup (NT threads; over more than kWaveTies entries with one LDS add per
// wave and bin, hist_add, since a long list may be one run of equal keys, whose
// per-lane adds to one bin would serialise), and the entries that fall in
// the chosen digit are copied to sc by the whole workgroup; one wave then
// finishes over that short list (wave_threshold).  With more than
// kThrScratch entries in the chosen digit (or nothing to split on) the wave
// continues over the whole list, up to kWaveTies entries; beyond that the
// whole workgroup searches it (block_threshold), as one wave walking every
// digit of a long list -- a large group of equal scores at the cut -- is the
// slow case.  Every thread returns the threshold.  Contains workgroup
// barriers; sh_thr is LDS.
constexpr int kWaveTies = 2048;

template <int NT, class Get>
__device__ Threshold tie_threshold(const Get& get, int n, uint32_t need, SelectShared& sh,
                                   ThresholdScratch* sc, Threshold* sh_thr, uint64_t key_lo,
                                   uint64_t key_hi, int pos_bits) {
  const int tid = threadIdx.x;
  const int nb = (key_lo == key_hi) ? 0 : 64 - __clzll(key_lo ^ key_hi);
  const uint32_t need_all = need;
  if (nb > 0 && n > kThrScratch) {  // workgroup-uniform
    const int d = nb < 8 ? nb : 8;
    const int shft = nb - d;
    const uint64_t dmask = (1ull << d) - 1ull;
    const uint64_t top = (nb >= 64) ? 0ull : ((key_hi >> nb) << nb);  // bits every key shares
    for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
    if (tid == 0) sc->fill = 0;
    __syncthreads();
    if (n > kWaveTies) {  // a long list may be one run of equal keys
      for (int i0 = 0; i0 < n; i0 += NT) {  // whole waves: hist_add is per wave
        const int i = i0 + tid;
        uint64_t u;
        uint32_t p;
        get(min(i, n - 1), u, p);
        hist_add(sh.hist, (uint32_t)((u >> shft) & dmask), i < n);
      }
    } else {
      for (int i = tid; i < n; i += NT) {
        uint64_t u;
        uint32_t p;
        get(i, u, p);
        atomicAdd(&sh.hist[(uint32_t)((u >> shft) & dmask)], 1u);
      }
    }
    __syncthreads();
    find_crossing(sh, need, true);
    __syncthreads();
    const uint32_t beta = sh.beta, before = sh.before, cnt = sh.cnt;
    need -= before;
    const uint64_t prefix = top | ((uint64_t)beta << shft);
    const uint64_t low = (1ull << shft) - 1ull;
    if (cnt == need) return Threshold{prefix, 0u, 0};  // the whole digit is kept
    if (cnt <= (uint32_t)kThrScratch) {
      for (int i = tid; i < n; i += NT) {
        uint64_t u;
        uint32_t p;
        get(i, u, p);
        if ((u >> shft) == (prefix >> shft)) {
          const uint32_t k = atomicAdd(&sc->fill, 1u);  // k < cnt
          sc->key[k] = u;
          sc->pos[k] = p;
        }
      }
      __syncthreads();
      if (wave_id() == 0) {
        auto get_sc = [&](int i, uint64_t& u, uint32_t& p) {
          u = sc->key[i];
          p = sc->pos[i];
        };
        const Threshold t = wave_threshold(get_sc, (int)cnt, need, sh.hist, prefix, prefix | low,
                                           pos_bits);
        if (lane_id() == 0) *sh_thr = t;
      }
      __syncthreads();
      return *sh_thr;
    }
    if (cnt > (uint32_t)kWaveTies) return block_threshold<NT>(get, n, need_all, sh);
    key_lo = prefix;
    key_hi = prefix | low;
  }
  if (nb == 0 && n > kWaveTies) return block_threshold<NT>(get, n, need_all, sh);
  if (wave_id() == 0) {
    const Threshold t = wave_threshold(get, n, need, sh.hist, key_lo, key_hi, pos_bits);
    if (lane_id() == 0) *sh_thr = t;
  }
  __syncthreads();
  return *sh_thr;
}

}  // namespace ls
