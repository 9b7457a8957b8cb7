// Merge of per-shard top-k lists: the exchange step of indexer context
// parallelism, emulated on one GPU (gfx950).
//
// Page "vllm.models.minimax_m3.amd.mono.weights", _build_cp_qkv: every rank
// keeps all ranks' index-q heads, so each rank scores its share of every
// sequence's index pages for all heads; the candidates of a head then go to
// its owner, which keeps the head's top-k.  Here the G shard lists of a
// query token are merged by the selection rule of the index call: higher
// fp32 score first, ties to the lower position, NaN below every number.
//
// One workgroup per query token.  The G * k_in candidates become 64-bit keys
// (order-preserving score key << 32 | ~position; 0 for an empty slot), held
// in registers, 32 per thread.  Every key is distinct (a position sits in
// one shard only), so the k_out-th largest key K* is unique and the
// selection is exactly the keys >= K*.  K* is found by a radix select over
// the range the keys actually span: each pass cuts the current range
// [lo, hi] into at most 2048 bins of 2^s keys, counts the keys in each, and
// narrows the range to the bin holding the remaining rank; it stops as soon
// as that rank equals its bin's count (the whole bin is taken), at the
// latest when bins hold one key value.  Binning the span rather than fixed
// digits of the key spreads scores of one magnitude over many bins, so the
// LDS counters see little contention.  The selected keys are compacted with
// one LDS counter.
#include "block_ops.h"
#include "launch.h"
#include "mono_decode.h"

namespace mono {
namespace {

constexpr int kMergePer = 32;                         // candidates per thread
constexpr int kMergeMax = kMergePer * kBlock;         // 8192 per query token
constexpr int kDigitBins = 2048;

__device__ __forceinline__ float score_of_key(uint32_t key) {
  if (key == 0u) return __uint_as_float(0x7fc00000u);  // NaN scores map to key 0
  return (key & 0x80000000u) ? __uint_as_float(key & 0x7fffffffu) : __uint_as_float(~key);
}

struct MergeLds {
  uint32_t hist[kDigitBins];
  uint32_t scratch[kWaves + 3];
  uint64_t lo[kWaves], hi[kWaves];
};

__global__ __launch_bounds__(256) void topk_merge_kernel(const int32_t* __restrict__ cand_idx,
                                                         const float* __restrict__ cand_scores, int G, int N,
                                                         int k_in, int k_out, int32_t* __restrict__ out_idx,
                                                         float* __restrict__ out_scores) {
  __shared__ MergeLds lds;
  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  const int n = G * k_in;
  // Every load is issued before any is used (slots past the candidates
  // read the row's first one and are dropped below), so they all overlap.
  int32_t jv[kMergePer];
  float sv[kMergePer];
#pragma unroll
  for (int u = 0; u < kMergePer; ++u) {
    const int x = min(tid + kBlock * u, n - 1);
    const int g = x / k_in, c = x - g * k_in;
    const size_t off = ((size_t)g * N + i) * k_in + c;
    jv[u] = cand_idx[off];
    sv[u] = cand_scores[off];
  }
  uint64_t key[kMergePer];
  uint32_t n_mine = 0;
#pragma unroll
  for (int u = 0; u < kMergePer; ++u) {
    const bool ok = tid + kBlock * u < n && jv[u] >= 0;
    key[u] = ok ? ((uint64_t)score_key(sv[u]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)jv[u]) : 0ull;
    n_mine += ok;
  }
  uint32_t n_valid;
  (void)block_exclusive_scan(n_mine, lds.scratch, n_valid);

  // Threshold: keys >= thr are taken.
  uint64_t thr = 1;  // every non-empty key
  if (n_valid > (uint32_t)k_out) {
    // The span of the keys.
    uint64_t lo = ~0ull, hi = 0;
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) {
      if (key[u] != 0) {
        lo = key[u] < lo ? key[u] : lo;
        hi = key[u] > hi ? key[u] : hi;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint64_t ol = __shfl_xor(lo, off), oh = __shfl_xor(hi, off);
      lo = ol < lo ? ol : lo;
      hi = oh > hi ? oh : hi;
    }
    if ((tid & 63) == 0) {
      lds.lo[tid >> 6] = lo;
      lds.hi[tid >> 6] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      lo = lds.lo[w] < lo ? lds.lo[w] : lo;
      hi = lds.hi[w] > hi ? lds.hi[w] : hi;
    }
    uint32_t R = (uint32_t)k_out;
#pragma unroll 1
    for (;;) {
      const uint64_t width = hi - lo;
      const int bits = width == 0 ? 0 : 64 - __clzll((long long)width);
      const int shift = bits > 11 ? bits - 11 : 0;  // (width >> shift) < 2048
      for (int x = tid; x < kDigitBins; x += kBlock) lds.hist[x] = 0u;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kMergePer; ++u) {
        if (key[u] >= lo && key[u] <= hi && key[u] != 0) atomicAdd(&lds.hist[(uint32_t)((key[u] - lo) >> shift)], 1u);
      }
      __syncthreads();
      const BinSplit b = find_bin_of_rank(lds.hist, kDigitBins, R, lds.scratch);
      const uint64_t b_lo = lo + ((uint64_t)b.bin << shift);
      const uint64_t b_hi = shift == 0 ? b_lo : b_lo + (((uint64_t)1 << shift) - 1);
      R -= b.above;
      lo = b_lo;
      hi = b_hi < hi ? b_hi : hi;
      if (b.count == R || shift == 0) break;  // the whole bin is taken (one key value when shift == 0)
    }
    thr = lo;
  }
  // Each thread's taken keys go to consecutive slots after those of the
  // threads before it (one prefix sum).
  uint32_t n_take = 0;
#pragma unroll
  for (int u = 0; u < kMergePer; ++u) n_take += key[u] >= thr;  // thr >= 1: empty slots never count
  uint32_t n_taken;
  uint32_t slot = block_exclusive_scan(n_take, lds.scratch, n_taken);
#pragma unroll
  for (int u = 0; u < kMergePer; ++u) {
    if (key[u] >= thr) {
      if (slot < (uint32_t)k_out) {
        const size_t o = (size_t)i * k_out + slot;
        out_idx[o] = (int32_t)(0xFFFFFFFFu - (uint32_t)key[u]);
        if (out_scores) out_scores[o] = score_of_key((uint32_t)(key[u] >> 32));
      }
      ++slot;
    }
  }
  const uint32_t taken = min(n_taken, (uint32_t)k_out);
  for (int x = (int)taken + tid; x < k_out; x += kBlock) {
    const size_t o = (size_t)i * k_out + x;
    out_idx[o] = -1;
    if (out_scores) out_scores[o] = __uint_as_float(0x7fc00000u);
  }
}

}  // namespace

int launch_topk_merge(const int32_t* cand_idx, const float* cand_scores, int G, int N, int k_in, int k_out,
                      int32_t* out_idx, float* out_scores, hipStream_t stream) {
  if (G * k_in > kMergeMax) return set_error(MONO_ENOTSUP, "mono_topk_merge: more than %d candidates", kMergeMax);
  MONO_LAUNCH(kKTopkMerge, topk_merge_kernel, dim3(N), dim3(kBlock), 0, stream, cand_idx, cand_scores, G, N, k_in,
              k_out, out_idx, out_scores);
  return check_launch("mono_topk_merge");
}

}  // namespace mono
