// Paged GQA decode attention over MXFP4 K/V pages (or the older build's fp8
// pages, through the format policy of page_format.h): one split of one query
// token and KV head (gfx950).
//
// The pa_decode the mxfp4_pages page names reads [pages, heads, 8704] K and V
// pools as [pages, heads, 128, 64] data and [pages, heads, 128, 4] scales
// (page "vllm.models.minimax_m3.amd.ops.mxfp4_pages", mxfp4_page_views).
// Per query token: logits scale * q_h . k_j for the 16 query heads of a KV
// head over the candidate tokens (a selection list, or every token
// 0..pos), softmax, and the probability-weighted sum of the V rows.
//
// A split covers candidates [e0, e1); each wave takes groups of 16.  Per
// group, with lane (g = lane/16, m = lane%16):
//   * QK^T on bf16 MFMA 16x16x32 with the 16 *tokens* as M (lane (g, m)
//     loads the 16-byte chunk g of token m's K row, one e8m0 block) and the
//     16 query heads as N, so lane (g, n) ends with the logits of head n for
//     tokens 4g..4g+3 -- exactly the A-operand slots of a 16x16x16 MFMA;
//   * online softmax in the log2 domain (running max and sum per head);
//   * P V on bf16 MFMA 16x16x16 with heads as M and dims as N: the B operand
//     of lane (g, m) in tile x is dim 8m + x of tokens 4g..4g+3, so each lane
//     reads 4 bytes (dims 8m..8m+7) of four tokens' V rows straight from the
//     pool and no transpose through LDS is needed.
// The block-table row is staged in LDS before any wait, so token lookups
// cost one LDS read.  Dequantised K/V are exact in bf16, so the only
// roundings are fp32 accumulation, exp2, and the bf16 rounding of the
// probabilities (the row sums use the same rounded values).  Split partials
// (max, sum, 16x128 accumulator) are handed over with coherent stores; the
// last split to arrive merges them and writes the bf16 output.  The
// chunk-local instance (kLocal) reads its candidates from an LDS list and
// their pages from an LDS table instead of global memory.
#pragma once

#include "block_ops.h"
#include "launch.h"
#include "page_format.h"

#include <type_traits>

namespace mono {

constexpr int kGroupTokens = 16;
constexpr int kPassGroups = 4;  // groups of one wave whose entries are fetched together
constexpr int kBtCache = 4096;  // block-table entries staged in LDS (longer rows read global memory)
constexpr int kMergeBatch = 16;  // splits whose partials the merge requests at once (8 when 8 or fewer, and in the chunk-local step)
constexpr uint32_t kGateSpins = 1u << 21;  // bound of a gated split's wait (seconds)
// After the token loop the LDS holds the four waves' partial accumulators
// (32 KiB, [wave][head][dim]) and their running maxima and sums.
constexpr int kSoBytes = kWaves * kQHeads * kHeadDim * 4;
constexpr int kCombineBytes = kSoBytes + 2 * kWaves * kQHeads * 4 + 16;

struct AttnLds {
  union {
    int32_t bt[kBtCache];
    __attribute__((aligned(16))) uint8_t combine[kCombineBytes];
  };
};

struct AttnArgs {
  const uint16_t* q;        // this query token's 16 heads of KV head h: [16, 128]
  const uint8_t* k_pages;   // [num_pages, H, page bytes of the format]
  const uint8_t* v_pages;
  int64_t num_pages;
  int H, h;
  const int32_t* bt_row;    // block-table row of the request
  const int32_t* sel_row;   // selection list (coherent reads) or nullptr: dense
  int pos;                  // position of the query token
  int e0, e1;               // candidates of this split
  int split, n_splits;
  float scale;              // logit scale (times the K tensor scale for fp8)
  float v_scale;            // V tensor scale (1 for MXFP4)
  uint16_t* out;            // [16, 128] bf16 output of (query token, KV head)
  float* pm;                // [n_splits, 16] partial maxima of (query token, KV head)
  float* pl;                // [n_splits, 16] partial sums
  float* pacc;              // [n_splits, 2, 256, 4] partial accumulators (see the split's store)
  uint32_t* split_cnt;      // arrivals of (query token, KV head)
  uint32_t* err;
  // Gated splits only (else nullptr): the ready word of the split's (query
  // token, KV head), set once the token's selection is complete, which the
  // split waits for after its q and block-table loads and before reading
  // its entries; and the control block (a wait that runs out drops its
  // zero record).
  const uint32_t* sel_ready;
  uint32_t* ctrl;
  // Chunk-local attention only: the candidates are LDS entries (token
  // tok0 + llist[e]) whose pages are lptab[(j >> 7) - page0].
  const __attribute__((address_space(3))) uint16_t* llist;
  const __attribute__((address_space(3))) int32_t* lptab;
  int tok0, page0;
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_bf16x8(uint16_t* dst, const float* o, float inv) {
  u32x4_t w;
#pragma unroll
  for (int x = 0; x < 4; ++x) w[x] = bf16x2_bits(o[2 * x] * inv, o[2 * x + 1] * inv);
  *reinterpret_cast<u32x4_t*>(dst) = w;
}

// The K and V data of one group as one lane needs them.
template <class Fmt>
struct AttnGroup {
  typename Fmt::Chunk k;     // K chunk g (elements 32g..32g+31) of token m
  typename Fmt::Slice v[4];  // V elements 8m..8m+7 of tokens 4g..4g+3
  uint32_t vm;               // bit r: token r of the group is a candidate (the same in every lane)
};

// Returns true in the workgroup that wrote the output (the only split, or
// the last split to arrive, which merged the others).
// kGroups: groups of 16 tokens each wave fetches together in one pass (the
// attention-only kernel instance takes 2 to fit in fewer registers).
template <class Fmt, bool kLocal = false, int kGroups = kPassGroups>
__device__ __forceinline__ bool attn_split(const AttnArgs& a, AttnLds& lds) {
  const int tid = thread_index(), lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, m = lane & 15;
  const int e0 = a.e0, e1 = a.e1, pos = a.pos, H = a.H, h = a.h, split = a.split, n_splits = a.n_splits;
  const int n_groups = (e1 - e0 + kGroupTokens - 1) / kGroupTokens;
  MONO_STAMP(10);

  // The first pass's selection entries are requested first; the block-table
  // row (into LDS) and the q operand (into registers) load meanwhile.
  // Loaded values are never rewritten before use (a rewrite makes the
  // compiler wait for that load before issuing the next ones): entry loads
  // are unconditional, clamped inside the split, and whether an entry
  // counts is decided where it is used (token_of).
  auto entry_load = [&](int grp) -> int {
    const int entry = e0 + kGroupTokens * grp + m;
    if constexpr (kLocal) {
      return a.tok0 + (int)a.llist[max(0, min(entry, e1 - 1))];
    } else {
      if (!a.sel_row) return 0;
      return (int)load_coherent(reinterpret_cast<const uint32_t*>(a.sel_row + min(entry, e1 - 1)));
    }
  };
  auto token_of = [&](int grp, int raw) -> int {
    const int entry = e0 + kGroupTokens * grp + m;
    const bool in = grp < n_groups && entry < e1;
    return in ? ((kLocal || a.sel_row) ? raw : entry) : -1;
  };
  int jv[kGroups];
  const bool gated = !kLocal && a.sel_ready != nullptr;
  if (!gated) {
#pragma unroll
    for (int x = 0; x < kGroups; ++x) jv[x] = entry_load(wave + kWaves * x);
  }
  const int bt_len = (pos >> 7) + 1;
  const bool bt_lds = bt_len <= kBtCache;
  typedef __attribute__((address_space(3))) const int32_t lds_i32;
  lds_i32* const bt_local = (lds_i32*)(lds.bt);
  if (!kLocal && bt_lds)
    for (int x = tid; x < bt_len; x += kBlock) lds.bt[x] = a.bt_row[x];
  // B operand of QK^T: column n = m is query head m; k-slot (g, e) of k-step
  // s holds q element 32g + 8s + e.
  bf16x8_t qb[4];
  {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.q + (size_t)m * kHeadDim + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = __builtin_bit_cast(bf16x8_t, src[s]);
  }
  if (gated) {
    // The q operand and the block-table row load meanwhile.
    if (tid == 0) {
      uint32_t spins = 0;
      while (load_coherent(a.sel_ready) == 0u) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kGateSpins) {
          raise_error(a.err, kErrWait);
          store_coherent(a.ctrl + kHdrZeroed, 0u);
          break;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kGroups; ++x) jv[x] = entry_load(wave + kWaves * x);
  }
  __syncthreads();
  MONO_STAMP(11);

  const float sl2 = a.scale * 1.4426950408889634f;  // logits in log2 units
  // m_run: running maximum of head m (every lane (g, m)); acc[x][i] and
  // acc_l[i]: output dim 8m + x and softmax sum of head 4g + i.
  float m_run = -INFINITY;
  f32x4_t acc[8], acc_l = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const size_t kv_stride = (size_t)H * Fmt::kPageBytes;
  const uint8_t* kbase = a.k_pages + (size_t)h * Fmt::kPageBytes;
  const uint8_t* vbase = a.v_pages + (size_t)h * Fmt::kPageBytes;

  // Token j of lane (g, m) -> its pool row, packed as page << 7 | row, or
  // ~0u when it is not a candidate.  The page id comes from the LDS copy of
  // the block-table row through an LDS-qualified pointer, or, in the
  // long-table instance of the pass loop, from the row in global memory.
  // (A run-time choice between the two becomes one generic-address load,
  // whose wait covers both memory counters and so every K/V load in flight.)
  auto token_ref = [&](int j, auto long_table) -> uint32_t {
    if (j < 0 || j > pos) return ~0u;
    const int idx = j >> 7;
    int pid;
    if constexpr (kLocal) {
      pid = a.lptab[idx - a.page0];
    } else if constexpr (decltype(long_table)::value) {
      pid = a.bt_row[idx];
    } else {
      pid = bt_local[idx];
    }
    if (pid < 0 || pid >= a.num_pages) {
      raise_error(a.err, kErrPageId);
      return ~0u;
    }
    return ((uint32_t)pid << 7) | (uint32_t)(j & (kPageTokens - 1));
  };
  // Loads are unconditional and their values are not touched here.  A
  // non-candidate's K row is page 0, row 0: its logits become -inf in
  // qk_group (each logit depends on its own token's K row only).  Its V row
  // is that of the group's first candidate, so its V values are values the
  // group's candidates hold anyway, and its weight is exactly zero; a group
  // with no candidate skips P V (its V rows are page 0, row 0).  A NaN in a
  // row that is not a candidate's therefore cannot reach the output.
  auto load_group = [&](uint32_t ref) -> AttnGroup<Fmt> {
    AttnGroup<Fmt> t;
    const bool valid = ref != ~0u;
    const uint64_t bal = __ballot(valid);
    t.vm = (uint32_t)bal;  // lanes 0..15 hold tokens 0..15
    const uint32_t fb = bal ? (uint32_t)__builtin_amdgcn_readlane((int)ref, (int)__builtin_ctzll(bal)) : 0u;
    const uint32_t r0 = valid ? ref : 0u;
    {
      const uint8_t* page = kbase + (size_t)(r0 >> 7) * kv_stride;
      t.k = Fmt::load_chunk(page, Fmt::chunk_addr((int)(r0 & 127u), g));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ri = __shfl(ref, 4 * g + i);
      const uint32_t r1 = ri != ~0u ? ri : fb;
      const uint8_t* page = vbase + (size_t)(r1 >> 7) * kv_stride;
      t.v[i] = Fmt::load_slice(page, r1 & 127u, m);
    }
    return t;
  };
  // S^T tile of a group: lane (g, n) gets tokens 4g + i (i = 0..3) of head n.
  auto qk_group = [&](const AttnGroup<Fmt>& t) -> f32x4_t {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Fmt::chunk_bf16(t.k, s), qb[s], c, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = ((t.vm >> (4 * g + i)) & 1u) ? c[i] * sl2 : -INFINITY;
    return c;
  };
  // acc += P V and acc_l += P 1 of a group; pa is the A operand (row n =
  // head n, k-slot (g, i) = token 4g + i).
  auto pv_group = [&](const AttnGroup<Fmt>& t, s16x4_t pa) {
    if (t.vm == 0u) return;  // no candidate: every weight is zero
    // V of tokens 4g..4g+3, dims 8m..8m+7, as bf16 pairs (dims 8m+2p, 8m+2p+1).
    u32x4_t vv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = Fmt::slice_bf16(t.v[i]);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int p = x >> 1;
      // tokens (0, 1) and (2, 3) of dim 8m + x: low or high halves of the pairs
      const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t b01 = __builtin_amdgcn_perm(vv[1][p], vv[0][p], sel);
      const uint32_t b23 = __builtin_amdgcn_perm(vv[3][p], vv[2][p], sel);
      const s16x4_t vb = __builtin_bit_cast(s16x4_t, (uint64_t)b01 | ((uint64_t)b23 << 32));
      acc[x] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, acc[x], 0, 0, 0);
    }
    // The softmax sums: P times a column of bf16 ones.
    const s16x4_t ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80};
    acc_l = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, ones, acc_l, 0, 0, 0);
  };

  // A pass covers kGroups groups of this wave: page lookups, the K/V
  // loads of all of them at once, QK^T of all, one online-softmax update,
  // then P V of all.  The first pass's entries were requested at the start.
  auto passes = [&](auto long_table) {
  for (int gb = wave; gb < n_groups; gb += kWaves * kGroups) {
    AttnGroup<Fmt> grp[kGroups];
#pragma unroll
    for (int x = 0; x < kGroups; ++x) grp[x] = load_group(token_ref(token_of(gb + kWaves * x, jv[x]), long_table));
    // The next pass's entries load while this pass computes.
#pragma unroll
    for (int x = 0; x < kGroups; ++x) jv[x] = entry_load(gb + kWaves * kGroups + kWaves * x);
    f32x4_t z[kGroups];
    float mx = -INFINITY;
#pragma unroll
    for (int x = 0; x < kGroups; ++x) {
      z[x] = qk_group(grp[x]);
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[x][i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    // Rescale only when some head's maximum grew past a finite one (a head
    // whose maximum was -inf has had only zero weights so far).
    if (__ballot(alpha != 1.f && m_run != -INFINITY)) {
      // The accumulator rows are heads 4g..4g+3: their rescale factors sit
      // in lanes 4g..4g+3.
      f32x4_t al;
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[x] *= al;
      acc_l *= al;
    }
    m_run = m_new;
#pragma unroll
    for (int x = 0; x < kGroups; ++x) {
      const uint32_t p01 = bf16x2_bits(__builtin_amdgcn_exp2f(z[x][0] - m_use), __builtin_amdgcn_exp2f(z[x][1] - m_use));
      const uint32_t p23 = bf16x2_bits(__builtin_amdgcn_exp2f(z[x][2] - m_use), __builtin_amdgcn_exp2f(z[x][3] - m_use));
      pv_group(grp[x], __builtin_bit_cast(s16x4_t, (uint64_t)p01 | ((uint64_t)p23 << 32)));
    }
  }
  };
  if (kLocal || bt_lds) {
    passes(std::false_type{});
  } else {
    passes(std::true_type{});
  }

  // ---- combine the four waves -------------------------------------------
  __syncthreads();
  MONO_STAMP(12);  // the block-table copy is no longer read
  float* so = reinterpret_cast<float*>(lds.combine);  // [wave][head][dim]
  float(*s_m)[kQHeads] = reinterpret_cast<float(*)[kQHeads]>(lds.combine + kSoBytes);
  float(*s_l)[kQHeads] = reinterpret_cast<float(*)[kQHeads]>(lds.combine + kSoBytes + kWaves * kQHeads * 4);
  uint32_t* s_last = reinterpret_cast<uint32_t*>(lds.combine + kSoBytes + 2 * kWaves * kQHeads * 4);
  // acc[x][i] is head 4g + i, dim 8m + x.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* dst = so + wave * 2048 + (4 * g + i) * kHeadDim + 8 * m;
    *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
    *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
  }
  if (g == 0) s_m[wave][m] = m_run;
  if (m == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s_l[wave][4 * g + i] = acc_l[i];
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
    const float* src = so + w * 2048 + hd * kHeadDim + d0;
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] += src[x] * f;
  }

  uint16_t* orow = a.out + (size_t)hd * kHeadDim + d0;
  if (n_splits == 1) {
    store_bf16x8(orow, o, lsum > 0.f ? a.v_scale / lsum : 0.f);
    return true;
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
    // The accumulator slot of a split is 2 x 256 units of 16 B: unit (u, t)
    // holds dims d0 + 4u .. d0 + 4u + 3 of head hd of thread t, so each
    // store instruction writes 4 KiB of whole lines.
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(pacc + slot * kQHeads * kHeadDim, kQHeads * kHeadDim * 4);
    store_coherent_x4(r, (uint32_t)tid * 16u, u32x4_t{__float_as_uint(o[0]), __float_as_uint(o[1]),
                                                      __float_as_uint(o[2]), __float_as_uint(o[3])});
    store_coherent_x4(r, (uint32_t)(kBlock + tid) * 16u, u32x4_t{__float_as_uint(o[4]), __float_as_uint(o[5]),
                                                                 __float_as_uint(o[6]), __float_as_uint(o[7])});
  }
  MONO_STAMP(13);
  wait_vmem();
  __syncthreads();
  MONO_STAMP(14);
  if (tid == 0) {
    const uint32_t prev = atomicAdd(a.split_cnt, 1u);
    *s_last = (prev == (uint32_t)(n_splits - 1)) ? 1u : 0u;
  }
  __syncthreads();
  MONO_STAMP(15);
  if (!*s_last) return false;

  // ---- last workgroup: merge the splits of this (query token, KV head) ----
  // All partials are requested at once (up to kMergeBatch splits a round
  // trip, or half as many when there are no more splits than that).  The
  // maxima and sums of two splits share cache lines, so they are read
  // coherently; each accumulator slot is written by one split only and read
  // by this workgroup only, so plain 16-byte loads are current.
  M = -INFINITY;
  lsum = 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x) o[x] = 0.f;
  auto merge = [&](auto batch) {
    constexpr int kB = decltype(batch)::value;
    for (int s0 = 0; s0 < n_splits; s0 += kB) {
      float mv[kB], lv[kB];
      f32x4_t av[kB][2];
      // Loaded values are not rewritten before all loads of the batch are
      // issued (a rewrite makes the compiler wait load by load); splits past
      // the last are masked where the values are used.
#pragma unroll
      for (int y = 0; y < kB; ++y) {
        const size_t sl = (size_t)min(s0 + y, n_splits - 1);
        mv[y] = load_coherent(pm + sl * kQHeads + hd);
        lv[y] = load_coherent(pl + sl * kQHeads + hd);
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(pacc + sl * kQHeads * kHeadDim);
        av[y][0] = src[tid];
        av[y][1] = src[kBlock + tid];
      }
      float Mb = M;
#pragma unroll
      for (int y = 0; y < kB; ++y) Mb = fmaxf(Mb, s0 + y < n_splits ? mv[y] : -INFINITY);
      const float Mu_b = (Mb == -INFINITY) ? 0.f : Mb;
      const float fo = __builtin_amdgcn_exp2f(M - Mu_b);  // rescale what was merged so far
      lsum *= fo;
#pragma unroll
      for (int x = 0; x < 8; ++x) o[x] *= fo;
#pragma unroll
      for (int y = 0; y < kB; ++y) {
        const float f = s0 + y < n_splits ? __builtin_amdgcn_exp2f(mv[y] - Mu_b) : 0.f;
        lsum += lv[y] * f;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          o[x] += av[y][0][x] * f;
          o[4 + x] += av[y][1][x] * f;
        }
      }
      M = Mb;
    }
  };
  if constexpr (kLocal) {
    merge(std::integral_constant<int, kMergeBatch / 2>{});  // the chunk-local step keeps its register budget
  } else if (n_splits > kMergeBatch / 2) {
    merge(std::integral_constant<int, kMergeBatch>{});
  } else {
    merge(std::integral_constant<int, kMergeBatch / 2>{});
  }
  store_bf16x8(orow, o, lsum > 0.f ? a.v_scale / lsum : 0.f);
  MONO_STAMP(16);
  return true;
}

}  // namespace mono
