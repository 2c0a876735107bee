// Monotone bucketing of int32 indexer scores, shared by the coarse scoring
// kernel (which histograms its scores) and the candidate selection (which
// filters by the threshold bucket).  Buckets are float-like: exact below
// 128 in magnitude, then 64 sub-buckets per power of two, so one bucket
// spans at most 1/64 of its scores' magnitude.
#pragma once

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

}  // namespace ls
