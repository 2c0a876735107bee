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

}  // namespace ls
