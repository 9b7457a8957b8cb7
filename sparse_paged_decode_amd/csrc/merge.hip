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
// selection is exactly the keys >= K*.  K* is found by radix select: digit
// passes of 11, 11, 11, 11, 10 and 10 bits from the top, each a histogram
// of the keys still matching the prefix found so far; the search stops as
// soon as the remaining rank equals its bin's count (then the whole bin is
// taken).  The selected keys are compacted with one LDS counter.
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
  uint32_t cnt;
};

__global__ __launch_bounds__(256) void topk_merge_kernel(const int32_t* __restrict__ cand_idx,
                                                         const float* __restrict__ cand_scores, int G, int N,
                                                         int k_in, int k_out, int32_t* __restrict__ out_idx,
                                                         float* __restrict__ out_scores) {
  __shared__ MergeLds lds;
  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  const int n = G * k_in;
  uint64_t key[kMergePer];
  uint32_t n_mine = 0;
#pragma unroll
  for (int u = 0; u < kMergePer; ++u) {
    const int x = tid + kBlock * u;
    uint64_t kk = 0;
    if (x < n) {
      const int g = x / k_in, c = x - g * k_in;
      const size_t off = ((size_t)g * N + i) * k_in + c;
      const int32_t j = cand_idx[off];
      if (j >= 0) kk = ((uint64_t)score_key(cand_scores[off]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
    }
    key[u] = kk;
    n_mine += kk != 0;
  }
  uint32_t n_valid;
  (void)block_exclusive_scan(n_mine, lds.scratch, n_valid);

  // Radix select of the threshold: keys k with (k & mask) >= prefix are taken.
  uint64_t prefix = 0, mask = 0;
  if (n_valid > (uint32_t)k_out) {
    uint32_t R = (uint32_t)k_out;
    int shift = 64;
#pragma unroll 1
    for (int p = 0; p < 6; ++p) {
      const int wd = p < 4 ? 11 : 10;
      shift -= wd;
      const int nbins = 1 << wd;
      for (int x = tid; x < nbins; x += kBlock) lds.hist[x] = 0u;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kMergePer; ++u) {
        if (key[u] != 0 && (key[u] & mask) == prefix)
          atomicAdd(&lds.hist[(uint32_t)(key[u] >> shift) & (uint32_t)(nbins - 1)], 1u);
      }
      __syncthreads();
      const BinSplit b = find_bin_of_rank(lds.hist, nbins, R, lds.scratch);
      prefix |= (uint64_t)b.bin << shift;
      mask |= (uint64_t)(nbins - 1) << shift;
      R -= b.above;
      if (b.count == R) break;  // the whole bin is taken
    }
  }

  if (tid == 0) lds.cnt = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kMergePer; ++u) {
    const bool take = key[u] != 0 && (key[u] & mask) >= prefix;
    const uint32_t slot = wave_append(take, &lds.cnt);
    if (take && slot < (uint32_t)k_out) {
      const size_t o = (size_t)i * k_out + slot;
      out_idx[o] = (int32_t)(0xFFFFFFFFu - (uint32_t)key[u]);
      if (out_scores) out_scores[o] = score_of_key((uint32_t)(key[u] >> 32));
    }
  }
  __syncthreads();
  const uint32_t taken = min(lds.cnt, (uint32_t)k_out);
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
