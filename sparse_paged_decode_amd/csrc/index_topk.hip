// Index scoring and top-k selection over MXFP4 index-key pages (gfx950).
//
// The mxfp4_pages page ("vllm.models.minimax_m3.amd.ops.mxfp4_pages", module
// docstring and mxfp4_page_views) names index scorers that read the
// single-head index-key pool as [pages, 128, 64] data and [pages, 128, 4]
// scales, without giving their rule.  The rule implemented here: the score
// of token j for query token i is the fp32 dot product of the bf16 index-q
// row i with the dequantised index-key row j, and the selection is the k
// highest scores among tokens 0..pos_i (ties to the lower token index).
//
// Two kernels:
//   index_scan  -- streams each request's index pages once for all of its
//                  query tokens, computes the scores with bf16 MFMA
//                  (16 token rows x up to 4 query columns, fp32 accumulate;
//                  every product of a bf16 and an MXFP4 value is exact), stores
//                  them in the workspace and builds a per-query histogram of
//                  the top 11 bits of the order-preserving score key.  The
//                  last workgroup of a request locates the bin that holds the
//                  k-th largest score.
//   topk_filter -- one workgroup per (query token, slice of 4096 scores):
//                  tokens in bins above that bin are selected outright,
//                  tokens in the bin become candidates.  The last workgroup of
//                  a query token finishes the selection inside the bin with
//                  two more radix passes (11 + 10 key bits); exact ties at the
//                  threshold go to the lowest token indices.
#include "block_ops.h"
#include "launch.h"

namespace mono {

constexpr int kScanChunkPages = 16;  // index pages per scan workgroup
constexpr int kHistBins = 2048;      // top 11 bits of the score key
constexpr int kHistShift = 21;
constexpr int kSlice = 4096;         // scores per filter workgroup
constexpr int kCandCap = 8192;       // candidates kept per query token

TopkLayout topk_layout(int B, int T, int bt_stride, int k) {
  (void)k;
  TopkLayout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t N = (size_t)B * T;
  l.q_groups = (T + 3) / 4;
  l.lcap = bt_stride * kPageTokens;
  l.err = take(256);
  l.seq_cnt = take((size_t)B * l.q_groups * 4);
  l.flt_cnt = take(N * 4);
  l.out_cnt = take(N * 4);
  l.cand_cnt = take(N * 4);
  l.meta = take(N * 16);
  l.hist = take(N * kHistBins * 4);
  l.scores = take(N * (size_t)l.lcap * 4);
  l.cand = take(N * (size_t)kCandCap * 8);
  l.total = off;
  return l;
}

namespace {

// grid (chunks of kScanChunkPages pages, B, query groups of 4); 256 threads.
// Wave w scores rows 32w..32w+31 of every page of the chunk as two 16-row
// MFMA tiles; lane (g = lane/16, m = lane%16) loads the 16-byte chunk g
// (elements 32g..32g+31, one e8m0 block) of row m of a tile.
template <int TQ>
__global__ __launch_bounds__(256) void index_scan_kernel(
    const uint16_t* __restrict__ index_q, const uint8_t* __restrict__ pages, int64_t num_pages,
    const int32_t* __restrict__ block_table, int bt_stride, const int32_t* __restrict__ seq_lens,
    int T, int k, uint8_t* __restrict__ ws, TopkLayout lay) {
  __shared__ uint32_t hist[TQ * kHistBins];
  __shared__ uint32_t scratch[8];
  __shared__ uint32_t s_last;

  const int chunk = blockIdx.x, b = blockIdx.y, qg = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, m = lane & 15;
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + lay.err);
  const int lcap = lay.lcap;

  const int L = seq_lens[b];
  if (L < T || L > lcap) {
    if (chunk == 0 && qg == 0 && tid == 0) raise_error(err, kErrSeqLen);
    return;
  }
  const int t0 = qg * 4;
  const int tq = min(TQ, T - t0);
  const int n_tok = L - T + t0 + tq;  // tokens seen by the group's last query token
  const int n_pages = (n_tok + kPageTokens - 1) / kPageTokens;
  const int nchunks = (n_pages + kScanChunkPages - 1) / kScanChunkPages;
  if (chunk >= nchunks) return;
  const int p_begin = chunk * kScanChunkPages;
  const int p_end = min(p_begin + kScanChunkPages, n_pages);

  // B operand: column n = m is query token t0 + m (zero when m >= tq);
  // its k-slot (g, e) of k-step s holds index-q element 32g + 8s + e.
  const bool has_q = m < tq;
  const int qi_lane = b * T + t0 + (has_q ? m : 0);
  bf16x8_t bq[4];
  {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(index_q + (size_t)qi_lane * kHeadDim + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t v = src[s];
      if (!has_q) v = u32x4_t{0u, 0u, 0u, 0u};
      bq[s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  const int my_pos = has_q ? (L - T + t0 + m) : -1;
  float* my_scores = reinterpret_cast<float*>(ws + lay.scores) + (size_t)qi_lane * lcap;

  for (int x = tid; x < TQ * kHistBins; x += kBlock) hist[x] = 0;
  __syncthreads();

  const int32_t* bt_row = block_table + (size_t)b * bt_stride;
  const int row0 = 32 * wave + m;  // tile 0 row; tile 1 is row0 + 16

  auto page_base = [&](int p) -> const uint8_t* {
    int pid = bt_row[p];
    if (pid < 0 || pid >= num_pages) {
      raise_error(err, kErrPageId);
      pid = 0;
    }
    return pages + (size_t)pid * kPageBytes;
  };

  const uint8_t* pg = page_base(p_begin);
  u32x4_t d0 = *reinterpret_cast<const u32x4_t*>(pg + row0 * kRowBytes + 16 * g);
  u32x4_t d1 = *reinterpret_cast<const u32x4_t*>(pg + (row0 + 16) * kRowBytes + 16 * g);
  uint32_t e0 = pg[kScaleOffset + row0 * 4 + g];
  uint32_t e1 = pg[kScaleOffset + (row0 + 16) * 4 + g];

  for (int p = p_begin; p < p_end; ++p) {
    u32x4_t nd0 = d0, nd1 = d1;
    uint32_t ne0 = e0, ne1 = e1;
    if (p + 1 < p_end) {  // prefetch the next page while this one is scored
      const uint8_t* np = page_base(p + 1);
      nd0 = *reinterpret_cast<const u32x4_t*>(np + row0 * kRowBytes + 16 * g);
      nd1 = *reinterpret_cast<const u32x4_t*>(np + (row0 + 16) * kRowBytes + 16 * g);
      ne0 = np[kScaleOffset + row0 * 4 + g];
      ne1 = np[kScaleOffset + (row0 + 16) * 4 + g];
    }
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const u32x4_t d = tile ? d1 : d0;
      const float sc = e8m0_scale_operand(tile ? e1 : e0);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8_bf16(d[s], sc), bq[s], acc, 0, 0, 0);
      // acc[i] of lane (g, m): row 4g + i of the tile, query column m
      if (has_q) {
        const int j0 = p * kPageTokens + 32 * wave + 16 * tile + 4 * g;
        if (j0 + 3 <= my_pos) {
          *reinterpret_cast<f32x4_t*>(my_scores + j0) = acc;
#pragma unroll
          for (int i = 0; i < 4; ++i) atomicAdd(&hist[m * kHistBins + (score_key(acc[i]) >> kHistShift)], 1u);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (j0 + i <= my_pos) {
              my_scores[j0 + i] = acc[i];
              atomicAdd(&hist[m * kHistBins + (score_key(acc[i]) >> kHistShift)], 1u);
            }
          }
        }
      }
    }
    d0 = nd0;
    d1 = nd1;
    e0 = ne0;
    e1 = ne1;
  }
  __syncthreads();

  uint32_t* ghist = reinterpret_cast<uint32_t*>(ws + lay.hist) + (size_t)(b * T + t0) * kHistBins;
  for (int x = tid; x < tq * kHistBins; x += kBlock) {
    const uint32_t v = hist[x];
    if (v) atomicAdd(&ghist[x], v);
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + lay.seq_cnt) + (size_t)b * lay.q_groups + qg;
    const uint32_t prev = atomicAdd(cnt, 1u);
    s_last = (prev == (uint32_t)(nchunks - 1)) ? 1u : 0u;
    if (s_last) *cnt = 0u;  // every arrival is in: leave the counter zero for the next call
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // Last workgroup of this request: locate the k-th largest score's bin.
  int4* meta = reinterpret_cast<int4*>(ws + lay.meta);
  for (int n = 0; n < tq; ++n) {
    const int qi = b * T + t0 + n;
    const int n_valid = L - T + t0 + n + 1;
    uint32_t* row = ghist + (size_t)n * kHistBins;
    if (n_valid <= k) {
      for (int x = tid; x < kHistBins; x += kBlock) row[x] = 0u;
      if (tid == 0) meta[qi] = make_int4(-1, 0, n_valid, 0);
      continue;
    }
    for (int x = tid; x < kHistBins; x += kBlock) hist[x] = load_coherent(&row[x]);
    __syncthreads();
    const BinSplit sp = find_bin_of_rank(hist, kHistBins, (uint32_t)k, scratch);
    for (int x = tid; x < kHistBins; x += kBlock) row[x] = 0u;
    if (tid == 0) meta[qi] = make_int4(sp.bin, (int)sp.above, n_valid, (int)sp.count);
    __syncthreads();
  }
}

struct Emitter {
  int32_t* out;
  float* out_scores;
  const float* scores;
  uint32_t k;
  uint32_t* err;
  // Slots past k would mean inconsistent counts; they are refused and flagged.
  __device__ __forceinline__ void put(uint32_t slot, int j) const {
    if (slot >= k) {
      raise_error(err, kErrSelection);
      return;
    }
    out[slot] = j;
    if (out_scores) out_scores[slot] = scores[j];
  }
};

// grid (B*T, slices of kSlice scores); 256 threads.
__global__ __launch_bounds__(256) void topk_filter_kernel(const int32_t* __restrict__ seq_lens, int T,
                                                          int k, uint8_t* __restrict__ ws,
                                                          TopkLayout lay, int32_t* __restrict__ sel_idx,
                                                          float* __restrict__ sel_scores) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t scratch[8];
  __shared__ uint32_t s_last;
  __shared__ uint32_t s_emit;

  const int i = blockIdx.x, slice = blockIdx.y, tid = threadIdx.x;
  const int b = i / T, t = i % T;
  const int lcap = lay.lcap;
  const int L = seq_lens[b];
  if (L < T || L > lcap) return;  // reported by the scan kernel
  const int n_valid = L - T + t + 1;
  const int n_slices = (n_valid + kSlice - 1) / kSlice;
  if (slice >= n_slices) return;

  const int4 mt = reinterpret_cast<const int4*>(ws + lay.meta)[i];
  const float* sc = reinterpret_cast<const float*>(ws + lay.scores) + (size_t)i * lcap;
  Emitter em{sel_idx + (size_t)i * k, sel_scores ? sel_scores + (size_t)i * k : nullptr, sc, (uint32_t)k,
             reinterpret_cast<uint32_t*>(ws + lay.err)};
  const int j0 = slice * kSlice, j1 = min(j0 + kSlice, n_valid);

  if (mt.x < 0) {  // at most k valid tokens: all of them, then -1 padding
    for (int j = j0 + tid; j < j1; j += kBlock) em.put((uint32_t)j, j);
    if (slice == 0) {
      for (int s = n_valid + tid; s < k; s += kBlock) {
        em.out[s] = -1;
        if (em.out_scores) em.out_scores[s] = __uint_as_float(0x7fc00000u);
      }
    }
    return;
  }

  const uint32_t B1 = (uint32_t)mt.x;
  const uint32_t above = (uint32_t)mt.y;
  const uint32_t in_bin = (uint32_t)mt.w;
  const bool use_cand = in_bin <= (uint32_t)kCandCap;
  uint32_t* out_cnt = reinterpret_cast<uint32_t*>(ws + lay.out_cnt) + i;
  uint32_t* cand_cnt = reinterpret_cast<uint32_t*>(ws + lay.cand_cnt) + i;
  uint2* cand = reinterpret_cast<uint2*>(ws + lay.cand) + (size_t)i * kCandCap;

  for (int jb = j0; jb < j1; jb += kBlock) {
    const int j = jb + tid;
    const bool in = j < j1;
    const uint32_t key = in ? score_key(sc[j]) : 0u;
    const uint32_t bin = key >> kHistShift;
    const bool hi = in && bin > B1;
    const bool eq = in && bin == B1;
    const uint32_t slot = wave_append(hi, out_cnt);
    if (hi) em.put(slot, j);
    if (use_cand) {
      const uint32_t cs = wave_append(eq, cand_cnt);
      if (eq && cs < (uint32_t)kCandCap) cand[cs] = make_uint2(key, (uint32_t)j);
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + lay.flt_cnt) + i;
    const uint32_t prev = atomicAdd(cnt, 1u);
    s_last = (prev == (uint32_t)(n_slices - 1)) ? 1u : 0u;
    if (s_last) *cnt = 0u;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- last workgroup of query i: pick the remaining R tokens of bin B1 ----
  const uint32_t R = (uint32_t)k - above;  // 1 <= R <= in_bin
  if (tid == 0) s_emit = above;
  // Candidate source: the compacted list, or (if it overflowed) every valid
  // score filtered by bin.  Both yield the same multiset of (key, j).
  const int n_src = use_cand ? (int)in_bin : n_valid;
  auto fetch = [&](int e, uint32_t& key, int& j) -> bool {
    if (use_cand) {
      const uint2 v = cand[e];
      key = v.x;
      j = (int)v.y;
      return true;
    }
    j = e;
    key = score_key(sc[e]);
    return (key >> kHistShift) == B1;
  };

  // pass 2: key bits 20..10
  for (int x = tid; x < kHistBins; x += kBlock) hist[x] = 0u;
  __syncthreads();
  for (int e = tid; e < n_src; e += kBlock) {
    uint32_t key;
    int j;
    if (fetch(e, key, j)) atomicAdd(&hist[(key >> 10) & 0x7FFu], 1u);
  }
  __syncthreads();
  const BinSplit s2 = find_bin_of_rank(hist, kHistBins, R, scratch);
  for (int e = tid; e < n_src; e += kBlock) {
    uint32_t key;
    int j;
    if (fetch(e, key, j) && ((key >> 10) & 0x7FFu) > (uint32_t)s2.bin) em.put(atomicAdd(&s_emit, 1u), j);
  }
  const uint32_t R2 = R - s2.above;
  const uint32_t pre2 = (B1 << 11) | (uint32_t)s2.bin;  // key >> 10 of the survivors

  // pass 3: key bits 9..0
  __syncthreads();
  for (int x = tid; x < 1024; x += kBlock) hist[x] = 0u;
  __syncthreads();
  for (int e = tid; e < n_src; e += kBlock) {
    uint32_t key;
    int j;
    if (fetch(e, key, j) && (key >> 10) == pre2) atomicAdd(&hist[key & 0x3FFu], 1u);
  }
  __syncthreads();
  const BinSplit s3 = find_bin_of_rank(hist, 1024, R2, scratch);
  const uint32_t kstar = (pre2 << 10) | (uint32_t)s3.bin;
  for (int e = tid; e < n_src; e += kBlock) {
    uint32_t key;
    int j;
    if (fetch(e, key, j) && (key >> 10) == pre2 && (key & 0x3FFu) > (uint32_t)s3.bin)
      em.put(atomicAdd(&s_emit, 1u), j);
  }
  const uint32_t R3 = R2 - s3.above;  // tokens to take among those with key == kstar

  if (s3.count == R3) {
    for (int e = tid; e < n_src; e += kBlock) {
      uint32_t key;
      int j;
      if (fetch(e, key, j) && key == kstar) em.put(atomicAdd(&s_emit, 1u), j);
    }
  } else {
    // More exact ties than places: take the lowest token indices, scanning
    // the scores in index order.
    __syncthreads();
    uint32_t taken = 0;
    for (int jb = 0; jb < n_valid && taken < R3; jb += kBlock) {
      const int j = jb + tid;
      const bool f = j < n_valid && score_key(sc[j]) == kstar;
      uint32_t tot;
      const uint32_t before = block_exclusive_scan(f ? 1u : 0u, scratch, tot);
      if (f && taken + before < R3) em.put(atomicAdd(&s_emit, 1u), j);
      taken += tot;
    }
  }
  if (tid == 0) {
    *out_cnt = 0u;
    *cand_cnt = 0u;
  }
}

}  // namespace

int launch_index_topk(const TopkArgs& a, const TopkLayout& lay, hipStream_t stream) {
  const dim3 g1((unsigned)((a.bt_stride + kScanChunkPages - 1) / kScanChunkPages), (unsigned)a.B,
                (unsigned)lay.q_groups);
  if (a.T == 1) {
    hipLaunchKernelGGL(index_scan_kernel<1>, g1, dim3(kBlock), 0, stream, a.index_q, a.pages,
                       a.num_pages, a.block_table, a.bt_stride, a.seq_lens, a.T, a.k, a.ws, lay);
  } else {
    hipLaunchKernelGGL(index_scan_kernel<4>, g1, dim3(kBlock), 0, stream, a.index_q, a.pages,
                       a.num_pages, a.block_table, a.bt_stride, a.seq_lens, a.T, a.k, a.ws, lay);
  }
  int rc = check_launch("mono_index_score_topk (scan)");
  if (rc) return rc;
  const dim3 g2((unsigned)(a.B * a.T), (unsigned)((lay.lcap + kSlice - 1) / kSlice));
  hipLaunchKernelGGL(topk_filter_kernel, g2, dim3(kBlock), 0, stream, a.seq_lens, a.T, a.k, a.ws, lay,
                     a.selected_idx, a.selected_scores);
  return check_launch("mono_index_score_topk (select)");
}

}  // namespace mono
