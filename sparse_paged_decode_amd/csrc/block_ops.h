// Workgroup-level helpers for 256-thread (4-wave) workgroups: prefix sums,
// wave-aggregated appends and the "which bin holds the R-th largest" search
// used by the radix top-k.
#pragma once

#include "device_common.h"

namespace mono {


__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Inclusive prefix sum within a 64-lane wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive prefix sum over the 256 threads in threadIdx order; `total`
// receives the sum of all values.  `scratch` is __shared__ uint32_t[kWaves].
// Must be reached by every thread of the workgroup.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch,
                                                         uint32_t& total) {
  const int wave = thread_index() >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane_id() == 63) scratch[wave] = incl;
  __syncthreads();
  uint32_t before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = scratch[w];
    before += (w < wave) ? s : 0u;
    sum += s;
  }
  __syncthreads();
  total = sum;
  return before + incl - v;
}

// Slot for each lane whose `pred` holds, taken from `*counter` with one
// atomic per wave.  Every lane of the wave must call it (convergent).
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return 0;
  const int lane = lane_id();
  const int leader = __ffsll((unsigned long long)mask) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
  base = __shfl(base, leader);
  return base + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
}

struct BinSplit {
  int bin;         // bin holding the R-th largest element
  uint32_t above;  // elements in bins above it (< R)
  uint32_t count;  // elements in that bin (above + count >= R)
};

// hist: __shared__ counts of `nbins` bins (nbins a multiple of 256, bins
// ordered by increasing key).  Finds the bin that holds the R-th largest
// element (1 <= R <= total count).  Every thread gets the result.
// `scratch` is __shared__ uint32_t[kWaves + 3].
__device__ __forceinline__ BinSplit find_bin_of_rank(const uint32_t* hist, int nbins, uint32_t R,
                                                     uint32_t* scratch) {
  if (thread_index() == 0) {  // defined result even if R exceeded the count
    scratch[kWaves] = 0u;
    scratch[kWaves + 1] = 0u;
    scratch[kWaves + 2] = 0u;
  }
  const int per = nbins / kBlock;
  // thread t owns the t-th group of `per` bins counted from the top
  const int hi = nbins - 1 - thread_index() * per;
  uint32_t sum = 0;
  for (int q = 0; q < per; ++q) sum += hist[hi - q];
  uint32_t total;
  uint32_t above = block_exclusive_scan(sum, scratch, total);
  if (above < R && R <= above + sum) {
    for (int q = 0; q < per; ++q) {
      const uint32_t c = hist[hi - q];
      if (above + c >= R) {
        scratch[kWaves] = (uint32_t)(hi - q);
        scratch[kWaves + 1] = above;
        scratch[kWaves + 2] = c;
        break;
      }
      above += c;
    }
  }
  __syncthreads();
  BinSplit r;
  r.bin = (int)scratch[kWaves];
  r.above = scratch[kWaves + 1];
  r.count = scratch[kWaves + 2];
  __syncthreads();
  return r;
}

}  // namespace mono
