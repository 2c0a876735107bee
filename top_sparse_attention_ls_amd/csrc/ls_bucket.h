// Monotone bucketing of indexer scores, shared by the kernels that
// histogram their scores (coarse scoring, prefill scoring, top-k) and the
// selections that filter by the threshold bucket.  Buckets are float-like:
// exact below 128 in magnitude, then 64 sub-buckets per power of two, so
// one bucket spans at most 1/64 of its scores' magnitude.  Two widths:
// int32 scores (3328 buckets) and int64 scores (7552 buckets).
#pragma once

#include "ls_device.h"
#include "ls_launch.h"

namespace ls {

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

// Scores that fall in magnitude bucket m: [lo, hi].
__device__ __forceinline__ void mag_range(uint32_t m, uint32_t& lo, uint32_t& hi) {
  if (m < 128u) {
    lo = hi = m;
    return;
  }
  const uint32_t e = 7u + (m - 128u) / 64u, j = (m - 128u) % 64u;
  lo = (64u + j) << (e - 6u);
  hi = lo + ((1u << (e - 6u)) - 1u);
}

// Scores that fall in bucket bk: [lo, hi] (the inverse of coarse_bucket).
__device__ __forceinline__ void coarse_bucket_range(int bk, int32_t& lo, int32_t& hi) {
  uint32_t a, b;
  if (bk >= kNBHalf) {
    mag_range((uint32_t)(bk - kNBHalf), a, b);
    lo = (int32_t)a;
    hi = (int32_t)b;
  } else {
    mag_range((uint32_t)(kNBHalf - 1 - bk), a, b);
    lo = -(int32_t)b - 1;
    hi = -(int32_t)a - 1;
  }
}

// ---- int64 scores
constexpr int kWideHalf = kWideBins / 2;  // magnitude buckets of a 63-bit value

__device__ __forceinline__ uint32_t wide_mag_bucket(uint64_t y) {  // y < 2^63
  if (y < 128u) return (uint32_t)y;
  const uint32_t e = 63u - (uint32_t)__clzll((long long)y);
  return 128u + (e - 7u) * 64u + (uint32_t)((y >> (e - 6u)) & 63u);
}

__device__ __forceinline__ void wide_mag_range(uint32_t m, uint64_t& lo, uint64_t& hi) {
  if (m < 128u) {
    lo = hi = m;
    return;
  }
  const uint32_t e = 7u + (m - 128u) / 64u, j = (m - 128u) % 64u;
  lo = (uint64_t)(64u + j) << (e - 6u);
  hi = lo + ((1ull << (e - 6u)) - 1ull);
}

// Monotone bucket of an int64 score in [0, kWideBins).
__device__ __forceinline__ uint32_t wide_bucket(int64_t x) {
  return x >= 0 ? (uint32_t)kWideHalf + wide_mag_bucket((uint64_t)x)
                : (uint32_t)kWideHalf - 1u - wide_mag_bucket((uint64_t)(-(x + 1)));
}

// Scores in bucket bk: [lo, hi] (the inverse of wide_bucket).
__device__ __forceinline__ void wide_bucket_range(int bk, int64_t& lo, int64_t& hi) {
  uint64_t a, b;
  if (bk >= kWideHalf) {
    wide_mag_range((uint32_t)(bk - kWideHalf), a, b);
    lo = (int64_t)a;
    hi = (int64_t)b;
  } else {
    wide_mag_range((uint32_t)(kWideHalf - 1 - bk), a, b);
    lo = -(int64_t)b - 1;
    hi = -(int64_t)a - 1;
  }
}

// Score kinds for the histogram-driven selections.
struct NarrowScore {  // int32 scores
  using T = int32_t;
  static constexpr int kBins = kCoarseBins;
  static __device__ __forceinline__ uint32_t bucket(T x) { return coarse_bucket(x); }
  static __device__ __forceinline__ void range(int bk, T& lo, T& hi) {
    coarse_bucket_range(bk, lo, hi);
  }
};
struct WideScore {  // int64 scores
  using T = int64_t;
  static constexpr int kBins = kWideBins;
  static __device__ __forceinline__ uint32_t bucket(T x) { return wide_bucket(x); }
  static __device__ __forceinline__ void range(int bk, T& lo, T& hi) {
    wide_bucket_range(bk, lo, hi);
  }
};

}  // namespace ls
