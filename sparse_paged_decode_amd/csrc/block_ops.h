// Workgroup-level helpers for 256-thread (4-wave) workgroups: prefix sums,
// wave-aggregated appends and the "which bin holds the R-th largest" search
// used by the radix top-k.
#pragma once

#include "device_common.h"

namespace mono {


__device__ __forceinline__ int lane_id() { return __lane_id(); }

// DPP controls (GFX9 encoding): shift right by n lanes within each row of
// 16, and broadcast lane 15 / lane 31 to the rows the row mask enables.
constexpr int kDppRowShr = 0x110;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// x of the lane the DPP control selects, or 0 where the source lane lies
// outside the row or the row mask leaves the lane's row out.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, kRowMask, 0xf, false);
}

// Inclusive prefix sum within a 64-lane wave, on DPP moves (no LDS round
// trips): a Hillis-Steele sum within each row of 16 lanes, then row 0's
// total added to row 1 and row 2's to row 3, then the first half's total
// to rows 2 and 3.  Every lane of the wave must be active.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += dpp_or_zero<kDppRowShr | 1, 0xf>(v);
  v += dpp_or_zero<kDppRowShr | 2, 0xf>(v);
  v += dpp_or_zero<kDppRowShr | 4, 0xf>(v);
  v += dpp_or_zero<kDppRowShr | 8, 0xf>(v);
  v += dpp_or_zero<kDppRowBcast15, 0xa>(v);
  v += dpp_or_zero<kDppRowBcast31, 0xc>(v);
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

constexpr int kMaxBinsPerThread = 8;  // find_bin_of_rank: histograms of up to 2048 bins

struct BinSplit {
  int bin;         // bin holding the R-th largest element
  uint32_t above;  // elements in bins above it (< R)
  uint32_t count;  // elements in that bin (above + count >= R)
};

// The split for per-thread bin counts in registers: thread t holds the
// counts of bins hi, hi - 1, ..., hi - per + 1 in h[0..per), where
// hi = nbins - 1 - t * per (groups of `per` bins counted from the top).
__device__ __forceinline__ BinSplit bin_of_rank_in_regs(const uint32_t (&h)[kMaxBinsPerThread], int per, int hi,
                                                        uint32_t R, uint32_t* scratch, uint32_t* total_out = nullptr) {
  if (thread_index() == 0) {  // defined result even if R exceeded the count
    scratch[kWaves] = 0u;
    scratch[kWaves + 1] = 0u;
    scratch[kWaves + 2] = 0u;
  }
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < kMaxBinsPerThread; ++q) sum += q < per ? h[q] : 0u;
  uint32_t total;
  uint32_t above = block_exclusive_scan(sum, scratch, total);
  if (total_out) *total_out = total;
  if (above < R && R <= above + sum) {
    int found = 0;
    uint32_t f_above = above, f_count = h[0];
#pragma unroll
    for (int q = kMaxBinsPerThread - 1; q >= 0; --q) {
      // bin q of the group holds the R-th largest when the bins before it
      // stay below R and it reaches R: exactly one q does
      uint32_t before = above;
#pragma unroll
      for (int p = 0; p < q; ++p) before += h[p];
      if (q < per && before < R && before + h[q] >= R) {
        found = q;
        f_above = before;
        f_count = h[q];
      }
    }
    scratch[kWaves] = (uint32_t)(hi - found);
    scratch[kWaves + 1] = f_above;
    scratch[kWaves + 2] = f_count;
  }
  __syncthreads();
  BinSplit r;
  r.bin = (int)scratch[kWaves];
  r.above = scratch[kWaves + 1];
  r.count = scratch[kWaves + 2];
  __syncthreads();
  return r;
}

// hist: __shared__ counts of `nbins` bins (nbins a multiple of 256, at most
// 2048, bins ordered by increasing key).  Finds the bin that holds the R-th
// largest element (1 <= R <= total count).  Every thread gets the result.
// `scratch` is __shared__ uint32_t[kWaves + 3].
__device__ __forceinline__ BinSplit find_bin_of_rank(const uint32_t* hist, int nbins, uint32_t R,
                                                     uint32_t* scratch) {
  const int per = nbins / kBlock;
  const int hi = nbins - 1 - thread_index() * per;
  uint32_t h[kMaxBinsPerThread];
#pragma unroll
  for (int q = 0; q < kMaxBinsPerThread; ++q) h[q] = q < per ? hist[hi - q] : 0u;
  return bin_of_rank_in_regs(h, per, hi, R, scratch);
}

// The same over a histogram row in global memory that other workgroups
// update (nbins 1024 or 2048): each thread reads its own group of bins with
// 16-byte coherent loads, straight into registers.  `total_out`, if given,
// receives the sum of the counts read (every thread the same).
template <int kBins>
__device__ __forceinline__ BinSplit find_bin_of_rank_global(const uint32_t* g, uint32_t R, uint32_t* scratch,
                                                            uint32_t* total_out = nullptr) {
  static_assert(kBins == 1024 || kBins == 2048, "four or eight bins per thread");
  constexpr int per = kBins / kBlock;
  const int hi = kBins - 1 - thread_index() * per;
  const int lo = hi - per + 1;
  const __amdgpu_buffer_rsrc_t rsrc = buffer_rsrc(g, (uint32_t)kBins * 4u);
  u32x4_t v[per / 4];
#pragma unroll
  for (int i = 0; i < per / 4; ++i) v[i] = load_coherent_x4(rsrc, (uint32_t)(lo + 4 * i) * 4u);
  uint32_t h[kMaxBinsPerThread];
#pragma unroll
  for (int q = 0; q < kMaxBinsPerThread; ++q) {
    const int x = per - 1 - q;  // bin hi - q is element x of the group
    h[q] = q < per ? v[x >> 2][x & 3] : 0u;
  }
  return bin_of_rank_in_regs(h, per, hi, R, scratch, total_out);
}

}  // namespace mono
