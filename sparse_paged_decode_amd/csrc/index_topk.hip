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
//                  (up to 4 query rows x 16 token columns, fp32 accumulate;
//                  every product of a bf16 and an MXFP4 value is exact), stores
//                  them in the workspace and builds a per-query histogram of
//                  the top 11 bits of the order-preserving score key.
//   topk_filter -- one workgroup per (query token, slice of 4096 scores):
//                  each finds the histogram bin that holds the k-th largest
//                  score; tokens in bins above it are selected outright,
//                  tokens in the bin become candidates.  The last workgroup of
//                  a query token finishes the selection inside the bin with
//                  two more radix passes (11 + 10 key bits); exact ties at the
//                  threshold go to the lowest token indices.
#include "block_ops.h"
#include "launch.h"

namespace mono {

constexpr int kScanChunkPages = 16;  // index pages per scan workgroup
constexpr int kBatch = 4;            // pages per prefetch batch
constexpr int kHistBins = 2048;      // top 11 bits of the score key
constexpr int kHistShift = 21;
constexpr int kSlice = 4096;         // scores per filter workgroup
constexpr int kCandCap = 8192;       // candidates kept per query token
constexpr int kLdsCand = 4096;       // candidates the resolving workgroup stages in LDS

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
  l.flt_cnt = take(N * 4);
  l.out_cnt = take(N * 4);
  l.cand_cnt = take(N * 4);
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
// (elements 32g..32g+31, one e8m0 block) of row m of a tile, which is the
// B-operand slot of that row's elements for the four k-steps.
template <int TQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void index_scan_kernel(
    const uint16_t* __restrict__ index_q, const uint8_t* __restrict__ pages, int64_t num_pages,
    const int32_t* __restrict__ block_table, int bt_stride, const int32_t* __restrict__ seq_lens,
    int T, uint8_t* __restrict__ ws, TopkLayout lay) {
  __shared__ uint32_t hist[TQ * kHistBins];

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

  // A operand: row m is query token t0 + m (zero when m >= tq); its k-slot
  // (g, e) of k-step s holds index-q element 32g + 8s + e.
  const bool has_q = m < tq;
  bf16x8_t aq[4];
  {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        index_q + (size_t)(b * T + t0 + (has_q ? m : 0)) * kHeadDim + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t v = src[s];
      if (!has_q) v = u32x4_t{0u, 0u, 0u, 0u};
      aq[s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // Scores and positions of the group's query tokens (used by lanes g == 0).
  float* q_scores = reinterpret_cast<float*>(ws + lay.scores) + (size_t)(b * T + t0) * lcap;
  const int pos0 = L - T + t0;  // position of query token t0; token t0 + i is at pos0 + i

  for (int x = tid; x < TQ * kHistBins; x += kBlock) hist[x] = 0;
  __syncthreads();

  const int32_t* bt_row = block_table + (size_t)b * bt_stride;
  const int row0 = 32 * wave + m;  // tile 0 row; tile 1 is row0 + 16
  // 32-bit lane offsets inside a page, so each load is (page base in SGPRs) +
  // (fixed lane offset) with no per-load address arithmetic.
  const uint32_t off_d0 = (uint32_t)(row0 * kRowBytes + 16 * g);
  const uint32_t off_d1 = off_d0 + 16u * kRowBytes;
  const uint32_t off_e0 = (uint32_t)(kScaleOffset + row0 * 4 + g);
  const uint32_t off_e1 = off_e0 + 16u * 4u;

  // The chunk's physical page ids, one per lane (lanes past the chunk repeat
  // its last page); each page's id is then taken with readlane, so no load
  // waits on a block-table lookup.
  const int n_cp = p_end - p_begin;
  int lane_pid = bt_row[p_begin + min(lane, n_cp - 1)];
  if (lane_pid < 0 || lane_pid >= num_pages) {
    raise_error(err, kErrPageId);
    lane_pid = 0;
  }

  // Pages are fetched in batches of kBatch, one batch ahead of the one being
  // scored.  Loads are unconditional (past the chunk end they repeat its last
  // page, whose rows are then all masked), so the compiler can count the
  // outstanding loads exactly and wait only for the batch being scored.
  struct Rows {
    u32x4_t d[2];
    uint32_t e[2];
  };
  auto load_batch = [&](Rows* r, int p0) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int cp = min(p0 + u - p_begin, n_cp - 1);
      const uint8_t* pg = pages + (size_t)__builtin_amdgcn_readlane(lane_pid, cp) * kPageBytes;
      r[u].d[0] = *reinterpret_cast<const u32x4_t*>(pg + off_d0);
      r[u].d[1] = *reinterpret_cast<const u32x4_t*>(pg + off_d1);
      r[u].e[0] = pg[off_e0];
      r[u].e[1] = pg[off_e1];
    }
  };
  // Scores of the wave's 32 rows of page p: C = Q K^T with the query tokens
  // as M and the 16 rows of a tile as N, so lane (g = 0, n) ends with the
  // scores of row n of the tile for query tokens 0..3 (acc[i]).  The two
  // tiles' MFMA chains are interleaved.
  auto score_page = [&](const Rows& r, int p) {
    const float sc0 = e8m0_scale_operand(r.e[0]);
    const float sc1 = e8m0_scale_operand(r.e[1]);
    f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[s], dequant8_bf16(r.d[0][s], sc0), c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[s], dequant8_bf16(r.d[1][s], sc1), c1, 0, 0, 0);
    }
    if (g == 0) {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const f32x4_t c = tile ? c1 : c0;
        const int j = p * kPageTokens + 32 * wave + 16 * tile + m;
#pragma unroll
        for (int i = 0; i < TQ; ++i) {
          if (i < tq && j <= pos0 + i) {
            q_scores[(size_t)i * lcap + j] = c[i];
            atomicAdd(&hist[i * kHistBins + (score_key(c[i]) >> kHistShift)], 1u);
          }
        }
      }
    }
  };

  // Two register sets used in turn (no copies between them, so a load never
  // has to wait for the registers it overwrites to drain).
  Rows ra[kBatch], rb[kBatch];
  load_batch(ra, p_begin);
  for (int p0 = p_begin; p0 < p_end; p0 += 2 * kBatch) {
    load_batch(rb, p0 + kBatch);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) score_page(ra[u], p0 + u);
    load_batch(ra, p0 + 2 * kBatch);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) score_page(rb[u], p0 + kBatch + u);
  }
  __syncthreads();

  uint32_t* ghist = reinterpret_cast<uint32_t*>(ws + lay.hist) + (size_t)(b * T + t0) * kHistBins;
  for (int x = tid; x < tq * kHistBins; x += kBlock) {
    const uint32_t v = hist[x];
    if (v) atomicAdd(&ghist[x], v);
  }
}

struct Emitter {
  int32_t* out;
  float* out_scores;
  const float* scores;
  uint32_t k;
  uint32_t* err;
  // Slots past k would mean inconsistent counts; they are refused and flagged.
  __device__ __forceinline__ void put(uint32_t slot, int j, float score) const {
    if (slot >= k) {
      raise_error(err, kErrSelection);
      return;
    }
    out[slot] = j;
    if (out_scores) out_scores[slot] = score;
  }
  __device__ __forceinline__ void put(uint32_t slot, int j) const {
    put(slot, j, out_scores ? scores[j] : 0.f);
  }
};

// grid (B*T, slices of kSlice scores); 256 threads.
__global__ __launch_bounds__(256) void topk_filter_kernel(const int32_t* __restrict__ seq_lens, int T,
                                                          int k, uint8_t* __restrict__ ws,
                                                          TopkLayout lay, int32_t* __restrict__ sel_idx,
                                                          float* __restrict__ sel_scores) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint2 s_cand[kLdsCand];
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

  const float* sc = reinterpret_cast<const float*>(ws + lay.scores) + (size_t)i * lcap;
  uint32_t* ghist = reinterpret_cast<uint32_t*>(ws + lay.hist) + (size_t)i * kHistBins;
  Emitter em{sel_idx + (size_t)i * k, sel_scores ? sel_scores + (size_t)i * k : nullptr, sc, (uint32_t)k,
             reinterpret_cast<uint32_t*>(ws + lay.err)};
  const int j0 = slice * kSlice, j1 = min(j0 + kSlice, n_valid);

  if (n_valid <= k) {  // at most k valid tokens: all of them, then -1 padding
    for (int j = j0 + tid; j < j1; j += kBlock) em.put((uint32_t)j, j);
    if (slice == 0) {
      for (int s = n_valid + tid; s < k; s += kBlock) {
        em.out[s] = -1;
        if (em.out_scores) em.out_scores[s] = __uint_as_float(0x7fc00000u);
      }
      for (int x = tid; x < kHistBins; x += kBlock) ghist[x] = 0u;  // unused; leave it zero
    }
    return;
  }

  // The bin of the k-th largest score, from the histogram the scan built.
  for (int x = tid; x < kHistBins; x += kBlock) hist[x] = ghist[x];
  __syncthreads();
  const BinSplit sp = find_bin_of_rank(hist, kHistBins, (uint32_t)k, scratch);
  const uint32_t B1 = (uint32_t)sp.bin;
  const uint32_t above = sp.above;
  const uint32_t in_bin = sp.count;
  const bool use_cand = in_bin <= (uint32_t)kCandCap;
  uint32_t* out_cnt = reinterpret_cast<uint32_t*>(ws + lay.out_cnt) + i;
  uint32_t* cand_cnt = reinterpret_cast<uint32_t*>(ws + lay.cand_cnt) + i;
  uint2* cand = reinterpret_cast<uint2*>(ws + lay.cand) + (size_t)i * kCandCap;

  // Load all of this thread's scores first, classify them, and reserve
  // output and candidate slots for the whole workgroup with one atomic each.
  constexpr int kPer = kSlice / kBlock;
  float v[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int j = j0 + q * kBlock + tid;
    v[q] = (j < j1) ? sc[j] : 0.f;
  }
  uint32_t hi_mask = 0, eq_mask = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int j = j0 + q * kBlock + tid;
    const uint32_t bin = score_key(v[q]) >> kHistShift;
    if (j < j1 && bin > B1) hi_mask |= 1u << q;
    if (j < j1 && bin == B1) eq_mask |= 1u << q;
  }
  // counts <= 4096 per workgroup, so both fit one packed 16+16-bit scan
  uint32_t tot;
  const uint32_t before = block_exclusive_scan(__popc(hi_mask) | (__popc(eq_mask) << 16), scratch, tot);
  if (tid == 0) {
    scratch[kWaves] = atomicAdd(out_cnt, tot & 0xFFFFu);
    scratch[kWaves + 1] = use_cand ? atomicAdd(cand_cnt, tot >> 16) : 0u;
  }
  __syncthreads();
  uint32_t slot = scratch[kWaves] + (before & 0xFFFFu);
  uint32_t cs = scratch[kWaves + 1] + (before >> 16);
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int j = j0 + q * kBlock + tid;
    if (hi_mask & (1u << q)) em.put(slot++, j, v[q]);
    if (use_cand && (eq_mask & (1u << q))) {
      if (cs < (uint32_t)kCandCap)
        store_coherent(reinterpret_cast<uint64_t*>(cand + cs),
                       ((uint64_t)(uint32_t)j << 32) | score_key(v[q]));
      ++cs;
    }
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + lay.flt_cnt) + i;
    const uint32_t prev = atomicAdd(cnt, 1u);
    s_last = (prev == (uint32_t)(n_slices - 1)) ? 1u : 0u;
    if (s_last) *cnt = 0u;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- last workgroup of query i: pick the remaining R tokens of bin B1 ----
  const uint32_t R = (uint32_t)k - above;  // 1 <= R <= in_bin
  if (tid == 0) s_emit = above;
  // Candidate source: the compacted list (staged in LDS when it fits), or,
  // if it overflowed, every valid score filtered by bin.  All three yield the
  // same multiset of (key, j).
  const bool in_lds = use_cand && in_bin <= (uint32_t)kLdsCand;
  if (in_lds) {
    for (int e = tid; e < (int)in_bin; e += kBlock) {
      const uint64_t c = load_coherent(reinterpret_cast<const uint64_t*>(cand + e));
      s_cand[e] = make_uint2((uint32_t)c, (uint32_t)(c >> 32));
    }
  }
  const int n_src = use_cand ? (int)in_bin : n_valid;
  auto fetch = [&](int e, uint32_t& key, int& j) -> bool {
    if (in_lds) {
      const uint2 c = s_cand[e];
      key = c.x;
      j = (int)c.y;
      return true;
    }
    if (use_cand) {
      const uint64_t c = load_coherent(reinterpret_cast<const uint64_t*>(cand + e));
      key = (uint32_t)c;
      j = (int)(c >> 32);
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
  for (int x = tid; x < kHistBins; x += kBlock) ghist[x] = 0u;  // every slice has read it
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
    MONO_LAUNCH(kKIndexScan, index_scan_kernel<1>, g1, dim3(kBlock), 0, stream, a.index_q, a.pages,
                       a.num_pages, a.block_table, a.bt_stride, a.seq_lens, a.T, a.ws, lay);
  } else {
    MONO_LAUNCH(kKIndexScan, index_scan_kernel<4>, g1, dim3(kBlock), 0, stream, a.index_q, a.pages,
                       a.num_pages, a.block_table, a.bt_stride, a.seq_lens, a.T, a.ws, lay);
  }
  int rc = check_launch("mono_index_score_topk (scan)");
  if (rc) return rc;
  const dim3 g2((unsigned)(a.B * a.T), (unsigned)((lay.lcap + kSlice - 1) / kSlice));
  MONO_LAUNCH(kKTopkFilter, topk_filter_kernel, g2, dim3(kBlock), 0, stream, a.seq_lens, a.T, a.k, a.ws, lay,
                     a.selected_idx, a.selected_scores);
  return check_launch("mono_index_score_topk (select)");
}

}  // namespace mono
