// The index scan on the matrix cores against the same scan on the vector
// ALUs, for benchmarks only (gfx950).
//
// Both kernels do the chunk-local step's scan phase: workgroup (b, c) scores
// pages [c * chunk_pages, ...) of request b for its one query token, keeps
// the scores in LDS, counts them in an LDS histogram of the top score-key
// bits and adds that histogram to hist[b] (global atomics).  Scores follow
// page "vllm.models.minimax_m3.amd.ops.mxfp4_pages" (module docstring): the
// dot product of the bf16 index query with each token's MXFP4 row, the row
// dequantised exactly to bf16 (e2m1 codes times the e8m0 block scale).
//   variant 0: the step's own scan_chunk (bf16 MFMA 16x16x32, the query as
//              row 0 of the A operand, two 16-token tiles per wave and page);
//   variant 1: v_dot2_f32_bf16 on the VALU: two lanes per token row, each
//              converting and multiplying 64 elements (32 packed pairs) and
//              adding its neighbour's half.
// The two differ only in how the 128 products of a token are summed in fp32.
#include "launch.h"
#include "topk_device.h"

namespace mono {
namespace {

constexpr int kScanLdsTokens = kLocalTokens;  // scores a workgroup keeps (32 pages)

struct BenchScanLds {
  ScanLds<1> scan;
  float scores[kScanLdsTokens];
  int32_t ptab[kMaxChunkPages];
};

// The pages of workgroup (b, c), or false when the request has none there.
// A length outside [1, bt_stride * 128] is flagged and the request skipped
// (its pages would lie past its block-table row).
__device__ __forceinline__ bool bench_chunk(const int32_t* seq_lens, int B, int bt_stride, int chunks,
                                            int chunk_pages, uint32_t* err, int& b, int& L, int& p_begin,
                                            int& p_end) {
  b = (int)blockIdx.x / chunks;
  const int c = (int)blockIdx.x % chunks;
  if (b >= B) return false;
  L = seq_lens[b];
  if (L < 1 || L > bt_stride * kPageTokens) {
    if (c == 0 && threadIdx.x == 0) raise_error(err, kErrSeqLen);
    return false;
  }
  const int n_pages = (L + kPageTokens - 1) / kPageTokens;
  p_begin = c * chunk_pages;
  p_end = min(p_begin + chunk_pages, n_pages);
  return p_begin < p_end;
}

__global__ __launch_bounds__(256) void scan_mfma_kernel(const uint16_t* index_q, const uint8_t* pages,
                                                        int64_t num_pages, const int32_t* block_table, int bt_stride,
                                                        const int32_t* seq_lens, int B, int chunks, int chunk_pages,
                                                        uint32_t* hist, uint32_t* err) {
  __shared__ BenchScanLds lds;
  int b, L, p_begin, p_end;
  if (!bench_chunk(seq_lens, B, bt_stride, chunks, chunk_pages, err, b, L, p_begin, p_end)) return;
  ScanArgs sa;
  sa.index_q = index_q;
  sa.pages = pages;
  sa.num_pages = num_pages;
  sa.bt_row = block_table + (size_t)b * bt_stride;
  sa.scores = nullptr;
  sa.ghist = hist;
  sa.err = err;
  sa.lcap = bt_stride * kPageTokens;
  sa.row[0] = sa.row[1] = sa.row[2] = sa.row[3] = b;
  sa.pos[0] = sa.pos[1] = sa.pos[2] = sa.pos[3] = L - 1;
  sa.tq = 1;
  sa.p_begin = p_begin;
  sa.p_end = p_end;
  scan_chunk<1, Mxfp4Format, true>(sa, lds.scan, (lds_f32*)lds.scores, (lds_i32w*)lds.ptab);
}

constexpr int kValuBatch = 2;  // pages a lane fetches ahead

__global__ __launch_bounds__(256) void scan_valu_kernel(const uint16_t* index_q, const uint8_t* pages,
                                                        int64_t num_pages, const int32_t* block_table, int bt_stride,
                                                        const int32_t* seq_lens, int B, int chunks, int chunk_pages,
                                                        uint32_t* hist, uint32_t* err) {
  __shared__ BenchScanLds lds;
  int b, L, p_begin, p_end;
  if (!bench_chunk(seq_lens, B, bt_stride, chunks, chunk_pages, err, b, L, p_begin, p_end)) return;
  const int tid = thread_index(), lane = tid & 63, wave = tid >> 6;
  const int half = lane & 1;            // elements 64 * half .. 64 * half + 63 of the row
  const int row = 32 * wave + (lane >> 1);
  const int pos = L - 1;

  // The query's 64 elements of this half as 32 bf16 pairs.
  uint32_t qv[32];
  {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(index_q + (size_t)b * kHeadDim + 64 * half);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const u32x4_t x = src[v];
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[4 * v + e] = x[e];
    }
  }
  for (int x = tid; x < kHistBins; x += kBlock) lds.scan.hist[x] = 0;
  const int n_cp = p_end - p_begin;
  int lane_pid = block_table[(size_t)b * bt_stride + p_begin + min(lane, n_cp - 1)];
  if (lane_pid < 0 || lane_pid >= num_pages) {
    raise_error(err, kErrPageId);
    lane_pid = 0;
  }
  __syncthreads();

  const uint32_t doff = (uint32_t)(row * kRowBytes + 32 * half);
  const uint32_t soff = (uint32_t)(kScaleOffset + row * 4);
  struct Row {
    u32x4_t d[2];  // 32 bytes: 64 codes
    uint32_t s;    // the row's four scale bytes
  };
  auto load_batch = [&](Row* r, int p0) {
#pragma unroll
    for (int u = 0; u < kValuBatch; ++u) {
      const int cp = min(p0 + u - p_begin, n_cp - 1);
      const uint8_t* pg = pages + (size_t)__builtin_amdgcn_readlane(lane_pid, cp) * Mxfp4Format::kPageBytes;
      r[u].d[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pg + doff));
      r[u].d[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pg + doff + 16));
      r[u].s = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(pg + soff));
    }
  };
  auto score_page = [&](const Row& r, int p) {
    if (p >= p_end) return;
    // Blocks 2 * half and 2 * half + 1 of the row: words 0..3 and 4..7.
    const float s0 = e8m0_scale_operand((r.s >> (16 * half)) & 0xFFu);
    const float s1 = e8m0_scale_operand((r.s >> (16 * half + 8)) & 0xFFu);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t word = r.d[w >> 2][w & 3];
      const float sc = w < 4 ? s0 : s1;
      const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0);
      const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1);
      const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2);
      const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3);
      acc = __builtin_amdgcn_fdot2_f32_bf16(p0, __builtin_bit_cast(bf16x2_t, qv[4 * w + 0]), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(p1, __builtin_bit_cast(bf16x2_t, qv[4 * w + 1]), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(p2, __builtin_bit_cast(bf16x2_t, qv[4 * w + 2]), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(p3, __builtin_bit_cast(bf16x2_t, qv[4 * w + 3]), acc, false);
    }
    const float s = acc + __shfl_xor(acc, 1);
    const int j = p * kPageTokens + row;
    if (half == 0 && j <= pos) {
      lds.scores[j - p_begin * kPageTokens] = s;
      atomicAdd(&lds.scan.hist[score_key(s) >> kHistShift], 1u);
    }
  };
  Row ra[kValuBatch], rb[kValuBatch];
  load_batch(ra, p_begin);
  for (int p0 = p_begin; p0 < p_end; p0 += 2 * kValuBatch) {
    load_batch(rb, p0 + kValuBatch);
#pragma unroll
    for (int u = 0; u < kValuBatch; ++u) score_page(ra[u], p0 + u);
    load_batch(ra, p0 + 2 * kValuBatch);
#pragma unroll
    for (int u = 0; u < kValuBatch; ++u) score_page(rb[u], p0 + kValuBatch + u);
  }
  __syncthreads();
  uint32_t* gh = hist + (size_t)b * kHistBins;
  for (int x = tid; x < kHistBins; x += kBlock) {
    const uint32_t v = lds.scan.hist[x];
    if (v) atomicAdd(&gh[x], v);
  }
}

}  // namespace

int launch_bench_scan(const uint16_t* index_q, const uint8_t* pages, int64_t num_pages, const int32_t* block_table,
                      int bt_stride, const int32_t* seq_lens, int B, int chunk_pages, int variant, uint32_t* hist,
                      uint32_t* err, hipStream_t stream) {
  const int chunks = (bt_stride + chunk_pages - 1) / chunk_pages;
  const dim3 grid((unsigned)(B * chunks));
  if (variant == 0) {
    MONO_LAUNCH(kKScanMfma, scan_mfma_kernel, grid, dim3(kBlock), 0, stream, index_q, pages, num_pages, block_table,
                bt_stride, seq_lens, B, chunks, chunk_pages, hist, err);
  } else {
    MONO_LAUNCH(kKScanValu, scan_valu_kernel, grid, dim3(kBlock), 0, stream, index_q, pages, num_pages, block_table,
                bt_stride, seq_lens, B, chunks, chunk_pages, hist, err);
  }
  return check_launch("mono_bench_scan");
}

}  // namespace mono
