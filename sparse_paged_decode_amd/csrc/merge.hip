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
// (order-preserving score key << 32 | ~position; 0 for an empty slot) in
// LDS, sorted in descending order by a bitonic network; the first k_out are
// the selection.  Every key is distinct (a position sits in one shard only),
// so the order is total.
#include "device_common.h"
#include "launch.h"

namespace mono {
namespace {

__device__ __forceinline__ float score_of_key(uint32_t key) {
  if (key == 0u) return __uint_as_float(0x7fc00000u);  // NaN scores map to key 0
  return (key & 0x80000000u) ? __uint_as_float(key & 0x7fffffffu) : __uint_as_float(~key);
}

__global__ __launch_bounds__(256) void topk_merge_kernel(const int32_t* __restrict__ cand_idx,
                                                         const float* __restrict__ cand_scores, int G, int N,
                                                         int k_in, int k_out, int n2, int32_t* __restrict__ out_idx,
                                                         float* __restrict__ out_scores) {
  extern __shared__ uint64_t keys[];  // n2 (a power of two >= G * k_in)
  const int i = blockIdx.x;
  const int n = G * k_in;
  for (int x = threadIdx.x; x < n2; x += blockDim.x) {
    uint64_t key = 0;
    if (x < n) {
      const int g = x / k_in, c = x - g * k_in;
      const size_t off = ((size_t)g * N + i) * k_in + c;
      const int32_t j = cand_idx[off];
      if (j >= 0) key = ((uint64_t)score_key(cand_scores[off]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
    }
    keys[x] = key;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (n2 >> 1); t += blockDim.x) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;  // direction of the run of `size` this pair sits in
        const uint64_t a = keys[lo], b = keys[hi];
        if (desc ? (a < b) : (a > b)) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int x = threadIdx.x; x < k_out; x += blockDim.x) {
    const uint64_t key = x < n2 ? keys[x] : 0ull;
    const size_t o = (size_t)i * k_out + x;
    out_idx[o] = key ? (int32_t)(0xFFFFFFFFu - (uint32_t)key) : -1;
    if (out_scores) out_scores[o] = key ? score_of_key((uint32_t)(key >> 32)) : __uint_as_float(0x7fc00000u);
  }
}

}  // namespace

int launch_topk_merge(const int32_t* cand_idx, const float* cand_scores, int G, int N, int k_in, int k_out,
                      int32_t* out_idx, float* out_scores, hipStream_t stream) {
  int n2 = 2;
  while (n2 < G * k_in) n2 <<= 1;
  MONO_LAUNCH(kKTopkMerge, topk_merge_kernel, dim3(N), dim3(256), (size_t)n2 * sizeof(uint64_t), stream, cand_idx,
              cand_scores, G, N, k_in, k_out, n2, out_idx, out_scores);
  return check_launch("mono_topk_merge");
}

}  // namespace mono
