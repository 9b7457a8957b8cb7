// Paged GQA decode attention over MXFP4 K/V pages: one split of one query
// token and KV head (gfx950).
//
// The pa_decode the mxfp4_pages page names reads [pages, heads, 8704] K and V
// pools as [pages, heads, 128, 64] data and [pages, heads, 128, 4] scales
// (page "vllm.models.minimax_m3.amd.ops.mxfp4_pages", mxfp4_page_views).
// Per query token: logits scale * q_h . k_j for the 16 query heads of a KV
// head over the candidate tokens (a selection list, or every token
// 0..pos), softmax, and the probability-weighted sum of the V rows.
//
// A split covers candidates [e0, e1); each wave takes groups of 32.  Per group:
//   * QK^T on bf16 MFMA 16x16x32 with the *tokens* as the M dimension (two
//     16-token tiles) and the 16 query heads as N, so each lane ends with the
//     logits of one head for 8 tokens -- exactly the B-operand layout the PV
//     product needs for the probabilities;
//   * online softmax in the log2 domain (running max and sum per head);
//   * PV as O^T = V^T P^T on the same MFMA: V is dequantised to bf16 and
//     written transposed into LDS (dims x token pairs), then read back 8
//     tokens per lane with one 16-byte LDS load per 16-dim tile.
// Dequantised K/V are exact in bf16, so the only roundings are fp32
// accumulation, exp2, and the bf16 rounding of the probabilities (the row
// sums use the same rounded values).  Split partials (max, sum, 16x128
// accumulator) are handed over with coherent stores; the last split to
// arrive merges them and writes the bf16 output.
#pragma once

#include "block_ops.h"
#include "launch.h"

namespace mono {

constexpr int kGroupTokens = 32;
constexpr int kVtRowBytes = 64;        // 16 token pairs x 4 B
constexpr int kVtRegionBytes = 8384;   // 128 rows + 3 x 64 B group pad, per wave
// After the token loop the same memory holds the four waves' partial
// accumulators (32 KiB) and their running maxima and sums.
constexpr int kSoBytes = kWaves * kQHeads * kHeadDim * 4;
static_assert(kSoBytes + 2 * kWaves * kQHeads * 4 + 4 <= kWaves * kVtRegionBytes, "attention LDS overlap");

struct AttnLds {
  __attribute__((aligned(16))) uint8_t vt[kWaves * kVtRegionBytes];
};

struct AttnArgs {
  const uint16_t* q;        // this query token's 16 heads of KV head h: [16, 128]
  const uint8_t* k_pages;   // [num_pages, H, 8704]
  const uint8_t* v_pages;
  int64_t num_pages;
  int H, h;
  const int32_t* bt_row;    // block-table row of the request
  const int32_t* sel_row;   // selection list (coherent reads) or nullptr: dense
  int pos;                  // position of the query token
  int e0, e1;               // candidates of this split
  int split, n_splits;
  float scale;
  uint16_t* out;            // [16, 128] bf16 output of (query token, KV head)
  float* pm;                // [n_splits, 16] partial maxima of (query token, KV head)
  float* pl;                // [n_splits, 16] partial sums
  float* pacc;              // [n_splits, 16, 128] partial accumulators
  uint32_t* split_cnt;      // arrivals of (query token, KV head)
  uint32_t* err;
};

// V^T element (dim, token pair) in a wave's region.  Rows are 64 B; the
// 16-byte chunk of a pair is XOR-swizzled by bits 2..3 of the row so the
// 16-row x 16-byte reads of one MFMA tile hit 64 distinct banks, and each
// group of 32 rows is shifted by 64 B so the four lane groups writing rows
// 32 apart do too.
__device__ __forceinline__ int vt_offset(int dim, int pair) {
  return dim * kVtRowBytes + (dim >> 5) * 64 + ((((pair >> 2) ^ (dim >> 2)) & 3) << 4) + (pair & 3) * 4;
}

__device__ __forceinline__ void store_bf16x8(uint16_t* dst, const float* o, float inv) {
  u32x4_t w;
#pragma unroll
  for (int x = 0; x < 4; ++x) w[x] = bf16x2_bits(o[2 * x] * inv, o[2 * x + 1] * inv);
  *reinterpret_cast<u32x4_t*>(dst) = w;
}

__device__ __forceinline__ void attn_split(const AttnArgs& a, AttnLds& lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, m = lane & 15;
  const int e0 = a.e0, e1 = a.e1, pos = a.pos, H = a.H, h = a.h, split = a.split, n_splits = a.n_splits;
  const int n_groups = (e1 - e0 + kGroupTokens - 1) / kGroupTokens;
  const int iters = (n_groups + kWaves - 1) / kWaves;

  // B operand of QK^T: column n = m is query head m; k-slot (g, e) of k-step
  // s holds q element 32g + 8s + e.
  bf16x8_t qb[4];
  {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.q + (size_t)m * kHeadDim + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = __builtin_bit_cast(bf16x8_t, src[s]);
  }
  const float sl2 = a.scale * 1.4426950408889634f;  // logits in log2 units
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t acc[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint8_t* vt = lds.vt + wave * kVtRegionBytes;

  // Groups are processed two at a time; the token lookups, block-table
  // lookups and K/V loads of both are issued before either is computed, so
  // each stage costs one memory round trip for the pair.
  struct Tok {
    u32x4_t kd, vd;
    uint32_t ke, ve;
    bool valid;
  };
  for (int it0 = 0; it0 < iters; it0 += 2) {
    Tok tk[2][2];
    int jj[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // lane (g, m) handles tokens 2m and 2m+1 of each 32-token group
        const int entry = e0 + kGroupTokens * (wave + kWaves * (it0 + x)) + 2 * m + u;
        int j = -1;
        if (it0 + x < iters && entry < e1) j = a.sel_row ? (int)load_coherent(reinterpret_cast<const uint32_t*>(a.sel_row + entry)) : entry;
        jj[x][u] = (j >= 0 && j <= pos) ? j : -1;
      }
    int pid[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int u = 0; u < 2; ++u) pid[x][u] = jj[x][u] >= 0 ? a.bt_row[jj[x][u] >> 7] : -1;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        Tok& t = tk[x][u];
        t.kd = t.vd = u32x4_t{0u, 0u, 0u, 0u};
        t.ke = t.ve = 127u;
        t.valid = false;
        const int j = jj[x][u];
        if (j >= 0) {
          if (pid[x][u] < 0 || pid[x][u] >= a.num_pages) {
            raise_error(a.err, kErrPageId);
          } else {
            const size_t off = ((size_t)pid[x][u] * H + h) * kPageBytes;
            const int r = j & (kPageTokens - 1);
            t.kd = *reinterpret_cast<const u32x4_t*>(a.k_pages + off + r * kRowBytes + 16 * g);
            t.vd = *reinterpret_cast<const u32x4_t*>(a.v_pages + off + r * kRowBytes + 16 * g);
            t.ke = a.k_pages[off + kScaleOffset + r * 4 + g];
            t.ve = a.v_pages[off + kScaleOffset + r * 4 + g];
            t.valid = true;
          }
        }
      }
#pragma unroll
  for (int xi = 0; xi < 2; ++xi) {
    if (it0 + xi >= iters) break;  // uniform across the workgroup
    u32x4_t kd[2] = {tk[xi][0].kd, tk[xi][1].kd}, vd[2] = {tk[xi][0].vd, tk[xi][1].vd};
    uint32_t ke[2] = {tk[xi][0].ke, tk[xi][1].ke}, ve[2] = {tk[xi][0].ve, tk[xi][1].ve};
    bool valid[2] = {tk[xi][0].valid, tk[xi][1].valid};

    // S^T tiles: lane (g, n) gets tokens 8g + 2i + u (i = 0..3) of head n.
    f32x4_t c[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float sc = e8m0_scale_operand(ke[u]);
      c[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        c[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8_bf16(kd[u][s], sc), qb[s], c[u], 0, 0, 0);
    }
    // Validity of token 2r + u sits in bit r of these ballots (lanes 0..15).
    const uint32_t vm0 = (uint32_t)__ballot(valid[0]);
    const uint32_t vm1 = (uint32_t)__ballot(valid[1]);
    float z[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t vm = u ? vm1 : vm0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool v = (vm >> (4 * g + r)) & 1u;
        z[u][r] = v ? c[u][r] * sl2 : -INFINITY;
        mx = fmaxf(mx, z[u][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    u32x4_t pw;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pw[r] = bf16x2_bits(__builtin_amdgcn_exp2f(z[0][r] - m_use), __builtin_amdgcn_exp2f(z[1][r] - m_use));
      psum += bf16_lo_to_f32(pw[r]) + bf16_hi_to_f32(pw[r]);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] *= alpha;
    // k-slot (g, e) of P^T is token 8g + e, e = 2r + u.
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);

    // V^T into LDS: row = dim, column = token pair m (tokens 2m, 2m+1).
    {
      const float sv0 = e8m0_scale_operand(ve[0]);
      const float sv1 = e8m0_scale_operand(ve[1]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4_t w0 = __builtin_bit_cast(u32x4_t, dequant8_bf16(vd[0][s], sv0));
        const u32x4_t w1 = __builtin_bit_cast(u32x4_t, dequant8_bf16(vd[1][s], sv1));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int d = 32 * g + 8 * s + 2 * q;
          *reinterpret_cast<uint32_t*>(vt + vt_offset(d, m)) = (w0[q] & 0xffffu) | (w1[q] << 16);
          *reinterpret_cast<uint32_t*>(vt + vt_offset(d + 1, m)) = (w0[q] >> 16) | (w1[q] & 0xffff0000u);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      // A operand: row m is dim 16x + m, k-slot (g, e) is token 8g + e.
      const bf16x8_t va =
          __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(vt + vt_offset(16 * x + m, 4 * g)));
      acc[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[x], 0, 0, 0);
    }
    __syncthreads();
  }
  }

  // ---- combine the four waves -------------------------------------------
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  float* so = reinterpret_cast<float*>(lds.vt);  // [wave][dim][head], 8 KiB per wave
  float(*s_m)[kQHeads] = reinterpret_cast<float(*)[kQHeads]>(lds.vt + kSoBytes);
  float(*s_l)[kQHeads] = reinterpret_cast<float(*)[kQHeads]>(lds.vt + kSoBytes + kWaves * kQHeads * 4);
  uint32_t* s_last = reinterpret_cast<uint32_t*>(lds.vt + kSoBytes + 2 * kWaves * kQHeads * 4);
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) so[wave * 2048 + (16 * x + 4 * g + r) * kQHeads + m] = acc[x][r];
  if (g == 0) {
    s_m[wave][m] = m_run;
    s_l[wave][m] = l_run;
  }
  __syncthreads();
  const int hd = tid >> 4;         // query head within the group
  const int d0 = (tid & 15) * 8;   // first of this thread's 8 dims
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][hd]);
  float Mu = (M == -INFINITY) ? 0.f : M;
  float lsum = 0.f, o[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) o[x] = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float f = __builtin_amdgcn_exp2f(s_m[w][hd] - Mu);
    lsum += s_l[w][hd] * f;
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] += so[w * 2048 + (d0 + x) * kQHeads + hd] * f;
  }

  uint16_t* orow = a.out + (size_t)hd * kHeadDim + d0;
  if (n_splits == 1) {
    store_bf16x8(orow, o, lsum > 0.f ? 1.f / lsum : 0.f);
    return;
  }

  const size_t slot = (size_t)split;
  float* pm = a.pm;
  float* pl = a.pl;
  float* pacc = a.pacc;
  if ((tid & 15) == 0) {
    store_coherent(pm + slot * kQHeads + hd, M);
    store_coherent(pl + slot * kQHeads + hd, lsum);
  }
  {
    float* dst = pacc + (slot * kQHeads + hd) * kHeadDim + d0;
#pragma unroll
    for (int x = 0; x < 8; ++x) store_coherent(dst + x, o[x]);
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(a.split_cnt, 1u);
    *s_last = (prev == (uint32_t)(n_splits - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (!*s_last) return;

  // ---- last workgroup: merge the splits of this (query token, KV head) ----
  // (partials are read with coherent loads)
  // Splits are read four at a time so their loads overlap.
  const size_t s0 = 0;
  M = -INFINITY;
  for (int s = 0; s < n_splits; s += 4) {
    float mv[4];
#pragma unroll
    for (int y = 0; y < 4; ++y) mv[y] = (s + y < n_splits) ? load_coherent(pm + (s0 + s + y) * kQHeads + hd) : -INFINITY;
#pragma unroll
    for (int y = 0; y < 4; ++y) M = fmaxf(M, mv[y]);
  }
  Mu = (M == -INFINITY) ? 0.f : M;
  lsum = 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x) o[x] = 0.f;
  for (int s = 0; s < n_splits; s += 4) {
    float mv[4], lv[4], av[4][8];
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const bool in = s + y < n_splits;
      const size_t sl = s0 + s + (in ? y : 0);
      mv[y] = in ? load_coherent(pm + sl * kQHeads + hd) : -INFINITY;
      lv[y] = in ? load_coherent(pl + sl * kQHeads + hd) : 0.f;
      const float* src = pacc + (sl * kQHeads + hd) * kHeadDim + d0;
#pragma unroll
      for (int x = 0; x < 8; ++x) av[y][x] = in ? load_coherent(src + x) : 0.f;
    }
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const float f = __builtin_amdgcn_exp2f(mv[y] - Mu);
      lsum += lv[y] * f;
#pragma unroll
      for (int x = 0; x < 8; ++x) o[x] += av[y][x] * f;
    }
  }
  store_bf16x8(orow, o, lsum > 0.f ? 1.f / lsum : 0.f);
}

}  // namespace mono
