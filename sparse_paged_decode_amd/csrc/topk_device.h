// Device building blocks of index scoring and top-k selection (gfx950).
//
// The mxfp4_pages page ("vllm.models.minimax_m3.amd.ops.mxfp4_pages", module
// docstring and mxfp4_page_views) names index scorers that read the
// single-head index-key pool as [pages, 128, 64] data and [pages, 128, 4]
// scales, without giving their rule.  The rule implemented here: the score
// of token j for query token i is the fp32 dot product of the bf16 index-q
// row i with the dequantised index-key row j, and the selection is the k
// highest scores among tokens 0..pos_i (ties to the lower token index).
//
//   scan_chunk   -- one workgroup scores a chunk of a request's index pages
//                   for up to 4 of its query tokens on bf16 MFMA, stores the
//                   fp32 scores and adds them to per-query histograms of the
//                   top 11 bits of the order-preserving score key.
//   filter_slice  -- one workgroup per slice of a query token's scores: the
//                    histogram gives the bin of the k-th largest score,
//                    tokens above it are selected outright, tokens in it
//                    become candidates.
//   resolve_query -- once every slice is done: the remaining tokens of that
//                    bin by two more radix passes (11 + 10 key bits); exact
//                    ties at the threshold go to the lowest token indices.
//
// Scores, histograms and selections cross workgroups, so they are written
// and read with coherent (agent-scope) operations.  The scan is written over
// a page-format policy (page_format.h): MXFP4 pages, or the fp8 pages of
// the older build.
#pragma once

#include "block_ops.h"
#include "launch.h"
#include "page_format.h"

#include <type_traits>

namespace mono {


// A scan's LDS.  One row: one count per histogram bin.  Several rows: two
// 16-bit counts per word (a chunk holds at most 64 x 128 = 8192 tokens), and
// the scores of kStagePages pages per row, written out as whole lines every
// kStagePages pages so the scan loop itself issues no global store.
constexpr int kStagePages = 24;  // 12 and 18 measured slower; 24 needs 64 KiB of LDS, two workgroups still fit a CU
template <int TQ>
struct ScanLds {
  static constexpr bool kPacked = TQ > 1;
  uint32_t hist[kPacked ? TQ * kHistBins / 2 : TQ * kHistBins];
  float sc[kPacked ? TQ : 1][kPacked ? kStagePages * kPageTokens : 1];
};

// ---------------------------------------------------------------------------
// scan_chunk: pages [p_begin, p_end) of request b for up to four index rows
// of the request (query tokens, or (head, token) pairs).
// Wave w scores rows 32w..32w+31 of every page as two 16-row MFMA tiles; lane
// (g = lane/16, m = lane%16) loads chunk g (elements 32g..32g+31: one e8m0
// block of 16 bytes, or 32 fp8 bytes) of row m of a tile, which is that
// row's B-operand slot for the four k-steps.  Scores: C = Q K^T with the
// group's index rows as M and the 16 token rows of a tile as N, so lane
// (0, n) ends with token row n's scores for group rows 0..3 (acc[i]): one
// read of the page serves all of them.
// ---------------------------------------------------------------------------
struct ScanArgs {
  const uint16_t* index_q;  // bf16 [rows, 128]
  const uint8_t* pages;     // [num_pages, page bytes of the format]
  int64_t num_pages;
  const int32_t* bt_row;    // block-table row of request b
  float* scores;            // score rows, lcap apart
  uint32_t* ghist;          // histogram rows, kHistBins apart
  uint32_t* err;
  int lcap;
  int row[4];               // index rows of the group (q vector, score row, histogram row)
  int pos[4];               // their positions (relative to the window's first token)
  int tq;                   // rows in the group (1..4)
  int p_begin, p_end;       // pages of the chunk
};

typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) int32_t lds_i32w;

// With kLocal (one query row), the scores go to lds_scores (token j of the
// chunk at j - 128 * p_begin) instead of global memory, and the chunk's page
// ids to lds_ptab: the chunk-local step keeps them there, a one-row scan
// item writes them out whole after the chunk.
template <int TQ, class Fmt, bool kLocal = false>
__device__ __forceinline__ void scan_chunk(const ScanArgs& a, ScanLds<TQ>& lds, lds_f32* lds_scores = nullptr,
                                           lds_i32w* lds_ptab = nullptr) {
  static_assert(!kLocal || TQ == 1, "chunk-local scans hold one query token");
  static_assert(kLocal || TQ > 1, "one-row scans keep their scores in LDS");
  constexpr int kBatch = kLocal ? Fmt::kScanBatchLocal : Fmt::kScanBatchMulti;  // pages per prefetch batch
  const int tid = thread_index(), lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, m = lane & 15;

  // A operand: row m is group row m (zero when m >= tq); its k-slot (g, e)
  // of k-step s holds index-q element 32g + 8s + e.
  const bool has_q = m < a.tq;
  bf16x8_t aq[4];
  {
    // (Selected by value: the rows are uniform, each read at a fixed index.)
    const int r0 = __builtin_amdgcn_readfirstlane(a.row[0]), r1 = __builtin_amdgcn_readfirstlane(a.row[1]);
    const int r2 = __builtin_amdgcn_readfirstlane(a.row[2]), r3 = __builtin_amdgcn_readfirstlane(a.row[3]);
    const int qrow = m == 1 ? r1 : m == 2 ? r2 : m == 3 ? r3 : r0;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.index_q + (size_t)(has_q ? qrow : r0) * kHeadDim + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t v = src[s];
      if (!has_q) v = u32x4_t{0u, 0u, 0u, 0u};
      aq[s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  constexpr bool kPacked = ScanLds<TQ>::kPacked;
  static_assert(!kPacked || kLocal || kStagePages % (2 * kBatch) == 0, "sub-blocks end with loop iterations");
  constexpr int kRowWords = kPacked ? kHistBins / 2 : kHistBins;
  for (int x = tid; x < TQ * kRowWords; x += kBlock) lds.hist[x] = 0;
  __syncthreads();

  const int row0 = 32 * wave + m;  // tile 0 row; tile 1 is row0 + 16
  // 32-bit lane offsets inside a page, so each load is (page base in SGPRs) +
  // (fixed lane offset) with no per-load address arithmetic.
  const typename Fmt::ChunkAddr off0 = Fmt::chunk_addr(row0, g);
  const typename Fmt::ChunkAddr off1 = Fmt::chunk_addr(row0 + 16, g);

  // The chunk's physical page ids, one per lane (lanes past the chunk repeat
  // its last page); each page's id is then taken with readlane, so no load
  // waits on a block-table lookup.
  const int p_begin = a.p_begin, p_end = a.p_end;
  const int n_cp = p_end - p_begin;
  int lane_pid = a.bt_row[p_begin + min(lane, n_cp - 1)];
  if (lane_pid < 0 || lane_pid >= a.num_pages) {
    raise_error(a.err, kErrPageId);
    lane_pid = 0;
  }
  if constexpr (kLocal) {
    if (wave == 0 && lane < n_cp) lds_ptab[lane] = lane_pid;
  }

  // Pages are fetched in batches of kBatch, one batch ahead of the one being
  // scored.  Loads are unconditional (past the chunk end they repeat its last
  // page, and those slots are skipped when scoring), so the compiler can
  // count the outstanding loads exactly and wait only for the batch being
  // scored.
  struct Rows {
    typename Fmt::Chunk c[2];  // tiles 0 and 1
  };
  auto load_batch = [&](Rows* r, int p0) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int cp = min(p0 + u - p_begin, n_cp - 1);
      const uint8_t* pg = a.pages + (size_t)__builtin_amdgcn_readlane(lane_pid, cp) * Fmt::kPageBytes;
      r[u].c[0] = Fmt::load_chunk_stream(pg, off0);
      r[u].c[1] = Fmt::load_chunk_stream(pg, off1);
    }
  };
  auto score_page = [&](const Rows& r, int p) {
    if (p >= p_end) return;  // past the chunk: the registers hold a repeat of its last page
    f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[s], Fmt::chunk_bf16(r.c[0], s), c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[s], Fmt::chunk_bf16(r.c[1], s), c1, 0, 0, 0);
    }
    if (g == 0) {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const f32x4_t c = tile ? c1 : c0;
        const int j = p * kPageTokens + 32 * wave + 16 * tile + m;
#pragma unroll
        for (int i = 0; i < TQ; ++i) {
          if constexpr (kPacked) {
            // every row's slot is written (rows past tq are never written out)
            lds.sc[i][(p - p_begin) % kStagePages * kPageTokens + 32 * wave + 16 * tile + m] = c[i];
          }
          if (i < a.tq && j <= a.pos[i]) {
            if constexpr (kLocal) lds_scores[j - p_begin * kPageTokens] = c[i];
            const uint32_t bin = score_key(c[i]) >> kHistShift;
            if constexpr (kPacked) {
              atomicAdd(&lds.hist[i * kRowWords + (bin >> 1)], 1u << ((bin & 1u) << 4));
            } else {
              atomicAdd(&lds.hist[i * kHistBins + bin], 1u);
            }
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
    if constexpr (kPacked) {
      // A sub-block of pages is complete: its score lines go out (the
      // next batch's loads are already in flight ahead of these stores).
      const int done = min(p0 + 2 * kBatch, p_end);
      if ((done - p_begin) % kStagePages == 0 || done == p_end) {
        const int sp0 = p_begin + (done - p_begin - 1) / kStagePages * kStagePages;
        const uint32_t n_bytes = (uint32_t)(done - sp0) * kPageTokens * 4u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TQ; ++i) {
          if (i < a.tq) {
            const __amdgpu_buffer_rsrc_t rsrc =
                buffer_rsrc(a.scores + (size_t)a.row[i] * a.lcap + (size_t)sp0 * kPageTokens, n_bytes);
            const u32x4_t* src = reinterpret_cast<const u32x4_t*>(lds.sc[i]);
            for (uint32_t q = (uint32_t)tid; q * 16u < n_bytes; q += kBlock) store_coherent_x4(rsrc, q * 16u, src[q]);
          }
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < TQ; ++i) {
    if (i < a.tq) {
      uint32_t* gh = a.ghist + (size_t)a.row[i] * kHistBins;
      for (int x = tid; x < kRowWords; x += kBlock) {
        const uint32_t v = lds.hist[i * kRowWords + x];
        if constexpr (kPacked) {
          if (v & 0xFFFFu) atomicAdd(&gh[2 * x], v & 0xFFFFu);
          if (v >> 16) atomicAdd(&gh[2 * x + 1], v >> 16);
        } else {
          if (v) atomicAdd(&gh[x], v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Selection of one query token's top k over tokens 0..n_valid-1, in two
// steps.  filter_slice runs on every slice of kSlice scores: it finds the
// histogram bin B1 that holds the k-th largest score, writes the tokens of
// higher bins straight to the output and appends the tokens of bin B1 to a
// candidate list.  resolve_query runs once all slices are done: it picks the
// remaining tokens from the candidates with two more radix passes.
// ---------------------------------------------------------------------------
constexpr int kLdsCand = 3840;   // candidates the resolving workgroup stages in LDS

constexpr int kFilterStage = 6144;  // words a filter slice stages its outputs in

struct FilterLds {
  uint32_t stage[kFilterStage];  // positions above the threshold bin, then (key, position) candidates
  uint32_t scratch[8];
};

constexpr int kSelBatchesMax = 16;  // select_query batches (kSelectMax / (kBlock * 16))

struct ResolveLds {
  uint32_t hist[kHistBins];
  uint2 cand[kLdsCand + 1];  // + a spare entry for branch-free writes
  uint32_t scratch[8];
  uint32_t cnt;
  uint16_t marks[kSelBatchesMax][kBlock];  // select_query: tokens above the threshold bin
};
// pick_in_bin stages positions in hist and cand seen as one word array.
static_assert(offsetof(ResolveLds, hist) == 0 && offsetof(ResolveLds, cand) == sizeof(uint32_t) * kHistBins,
              "hist and cand are contiguous");

struct SelectArgs {
  const float* scores;  // the query token's scores (coherent), lcap floats
  int lcap;             // capacity of the score row (a multiple of 128)
  uint32_t* ghist;      // its histogram row
  int32_t* out;         // [k] selected token positions, then -1 padding
  float* out_scores;    // [k] or nullptr
  uint32_t* out_cnt;    // slots taken by filter items
  uint64_t* cand;       // [kCandCap] (key, j) candidates
  uint32_t* cand_cnt;   // candidates appended
  uint32_t* err;
  int n_valid;
  int k;
  int j_base;           // position of score 0 (the first token of the page window)
};

// Slots past k would mean inconsistent counts; they are refused and flagged.
__device__ __forceinline__ void put_selection(const SelectArgs& a, uint32_t slot, int j, float score) {
  if (slot >= (uint32_t)a.k) {
    raise_error(a.err, kErrSelection);
    return;
  }
  store_coherent(reinterpret_cast<uint32_t*>(a.out + slot), (uint32_t)(j + a.j_base));
  if (a.out_scores) store_coherent(a.out_scores + slot, score);
}

// Finds the bin of the k-th largest score in the query token's (complete)
// histogram row.
__device__ __forceinline__ BinSplit kth_bin(const SelectArgs& a, uint32_t* scratch) {
  return find_bin_of_rank_global<kHistBins>(a.ghist, (uint32_t)a.k, scratch);
}

// Slice [j0, j1) of the scores.  Returns the histogram split it used (the
// bin of the k-th largest score), which the resolve can reuse; count = 0 and
// above = k when every valid token is selected.  With kLds the slice's
// scores are lscores[0, j1 - j0) in LDS (a scan chunk's own, j1 - j0 <=
// kSlice), which the slice's LDS may overlap, and `known` is the split of
// the complete histogram row, already read.
template <bool kLds = false>
__device__ __forceinline__ BinSplit filter_slice(const SelectArgs& a, int j0, int j1, FilterLds& lds,
                                                 const lds_f32* lscores = nullptr, const BinSplit* known = nullptr) {
  const int tid = thread_index();
  if (a.n_valid <= a.k) {  // at most k valid tokens: all of them, then -1 padding
    for (int j = j0 + tid; j < j1; j += kBlock)
      put_selection(a, (uint32_t)j, j, !a.out_scores ? 0.f : kLds ? lscores[j - j0] : load_coherent(a.scores + j));
    if (j0 == 0) {
      for (int s = a.n_valid + tid; s < a.k; s += kBlock) {
        store_coherent(reinterpret_cast<uint32_t*>(a.out + s), 0xffffffffu);
        if (a.out_scores) store_coherent(a.out_scores + s, __uint_as_float(0x7fc00000u));
      }
    }
    return BinSplit{0, (uint32_t)a.k, 0u};
  }
  // The slice's scores are loaded unconditionally (indices clamped inside the
  // row's capacity, masked below) so the loads overlap the histogram's.
  constexpr int kPer = kSlice / kBlock;
  float v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if constexpr (kLds) {
      v[u] = j0 + u * kBlock + tid < j1 ? lscores[u * kBlock + tid] : 0.f;
    } else {
      v[u] = load_coherent(a.scores + min(j0 + u * kBlock + tid, a.lcap - 1));
    }
  }
  if constexpr (kLds) __syncthreads();  // every score is in registers before the slice's LDS is written
  const BinSplit sp = known ? *known : kth_bin(a, lds.scratch);
  const uint32_t B1 = (uint32_t)sp.bin;
  const bool use_cand = sp.count <= (uint32_t)kCandCap;

  uint32_t hi_mask = 0, eq_mask = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = j0 + u * kBlock + tid;
    const uint32_t bin = score_key(v[u]) >> kHistShift;
    hi_mask |= (j < j1 && bin > B1) ? (1u << u) : 0u;
    eq_mask |= (j < j1 && bin == B1) ? (1u << u) : 0u;
  }
  if (!use_cand) eq_mask = 0;
  // counts <= kSlice per workgroup: both fit one packed 16+16-bit scan
  uint32_t tot;
  const uint32_t before = block_exclusive_scan(__popc(hi_mask) | (__popc(eq_mask) << 16), lds.scratch, tot);
  const uint32_t n_hi = tot & 0xFFFFu, n_eq = tot >> 16;
  // The slice's block of output slots and of candidate slots; while those
  // atomics are in flight the outputs are staged in LDS at their offsets in
  // the block (positions, then (key, position) pairs), to be written to
  // consecutive slots by consecutive lanes.  Without room, or with scores
  // to write as well, each lane writes its own.
  const bool staged = !a.out_scores && n_hi + 2u * n_eq <= (uint32_t)kFilterStage;
  uint32_t base_hi = 0, base_c = 0;
  if (tid == 0) {
    base_hi = n_hi ? atomicAdd(a.out_cnt, n_hi) : 0u;
    base_c = n_eq ? atomicAdd(a.cand_cnt, n_eq) : 0u;
  }
  if (staged) {
    uint32_t o = before & 0xFFFFu, c = n_hi + 2u * (before >> 16);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t j = (uint32_t)(j0 + u * kBlock + tid);
      if (hi_mask & (1u << u)) lds.stage[o++] = j;
      if (eq_mask & (1u << u)) {
        lds.stage[c] = score_key(v[u]);
        lds.stage[c + 1] = j;
        c += 2;
      }
    }
  }
  if (tid == 0) {
    lds.scratch[kWaves] = base_hi;
    lds.scratch[kWaves + 1] = base_c;
  }
  __syncthreads();
  base_hi = lds.scratch[kWaves];
  base_c = lds.scratch[kWaves + 1];
  if (staged) {
    for (uint32_t q = tid; q < n_hi; q += kBlock) put_selection(a, base_hi + q, (int)lds.stage[q], 0.f);
    for (uint32_t q = tid; q < n_eq; q += kBlock) {
      const uint32_t cs = base_c + q;
      const uint32_t key = lds.stage[n_hi + 2u * q], j = lds.stage[n_hi + 2u * q + 1u];
      if (cs < (uint32_t)kCandCap) store_coherent(a.cand + cs, ((uint64_t)j << 32) | key);
    }
    return sp;
  }
  uint32_t slot = base_hi + (before & 0xFFFFu);
  uint32_t cs = base_c + (before >> 16);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = j0 + u * kBlock + tid;
    if (hi_mask & (1u << u)) put_selection(a, slot++, j, v[u]);
    if (eq_mask & (1u << u)) {
      if (cs < (uint32_t)kCandCap) store_coherent(a.cand + cs, ((uint64_t)(uint32_t)j << 32) | score_key(v[u]));
      ++cs;
    }
  }
  return sp;
}

// Where pick_in_bin reads the tokens of the threshold bin from: LDS pairs
// of (key, j), LDS pairs of (score bits, j), the candidate list, or the
// score row itself.
enum : int { kSrcLds = 0, kSrcList = 1, kSrcScores = 2, kSrcLdsBits = 3 };

// The float with key `key` (score_key's inverse on every key but NaN's 0).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// The remaining k - above tokens, all in histogram bin B1 (which holds
// in_bin tokens), by radix passes over key bits 20..10, then 9..0; exact
// ties at the threshold go to the lowest token indices.  Slots above..k-1
// of the output are filled.  With kSrcLds or kSrcLdsBits the candidates are
// in lds.cand[0..in_bin) already: each thread then holds its share of them
// in registers for the first pass, the tokens above the pass's threshold
// sub-bin get their slots from one prefix sum (their positions are staged
// in LDS and written to consecutive slots by consecutive lanes, unless
// scores are written too), and the sub-bin's own tokens (rarely more than a
// few) are compacted to the end of lds.cand and, when at most 256, ranked
// against one another by (key descending, index ascending), which picks
// the same tokens the last pass and the tie rule would.
__device__ __forceinline__ void pick_in_bin(const SelectArgs& a, ResolveLds& lds, uint32_t B1, uint32_t above,
                                            uint32_t in_bin, int src) {
  const int tid = thread_index();
  const int n_valid = a.n_valid;
  const bool lds_src = src == kSrcLds || src == kSrcLdsBits;
  const uint32_t R = (uint32_t)a.k - above;  // 1 <= R <= in_bin
  // every source but the score row holds in_bin entries
  int n_src = src == kSrcScores ? n_valid : (int)in_bin;
  int cbase = 0;  // first LDS candidate of the current pass
  // All three sources yield the same multiset of (key, j).
  auto fetch = [&](int e, uint32_t& key, int& j) -> bool {
    if (lds_src) {
      const uint2 c = lds.cand[cbase + e];
      key = src == kSrcLds ? c.x : score_key(__uint_as_float(c.x));
      j = (int)c.y;
      return true;
    }
    if (src == kSrcList) {
      const uint64_t c = load_coherent(a.cand + e);
      key = (uint32_t)c;
      j = (int)(c >> 32);
      return true;
    }
    j = e;
    key = score_key(load_coherent(a.scores + e));
    return (key >> kHistShift) == B1;
  };
  // The score written beside a token: its LDS bits, else the key's value
  // (NaN's key 0 excepted, whose bits are read back).
  auto score_of = [&](uint32_t key, uint32_t bits, int j) -> float {
    if (!a.out_scores) return 0.f;
    if (src == kSrcLdsBits) return __uint_as_float(bits);
    return (lds_src && key != 0u) ? key_value(key) : load_coherent(a.scores + j);
  };
  auto emit = [&](int j) {
    put_selection(a, atomicAdd(&lds.cnt, 1u), j, a.out_scores ? load_coherent(a.scores + j) : 0.f);
  };
  if (!lds_src && tid == 0) lds.cnt = above;
  __syncthreads();  // the caller's LDS candidates are written

  // pass 2: key bits 20..10
  BinSplit s2;
  if (lds_src) {
    constexpr int kPer = kLdsCand / kBlock;
    uint32_t kx[kPer], bx[kPer], jx[kPer];
    uint32_t valid = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = u * kBlock + tid;
      const uint2 c = lds.cand[min(e, kLdsCand - 1)];
      bx[u] = c.x;
      jx[u] = c.y;
      kx[u] = src == kSrcLds ? c.x : score_key(__uint_as_float(c.x));
      valid |= e < (int)in_bin ? (1u << u) : 0u;
    }
    for (int x = tid; x < kHistBins; x += kBlock) lds.hist[x] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (valid & (1u << u)) atomicAdd(&lds.hist[(kx[u] >> 10) & 0x7FFu], 1u);
    __syncthreads();
    s2 = find_bin_of_rank(lds.hist, kHistBins, R, lds.scratch);
    uint32_t hi = 0, eq = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t sub = (kx[u] >> 10) & 0x7FFu;
      hi |= ((valid >> u) & 1u) && sub > (uint32_t)s2.bin ? (1u << u) : 0u;
      eq |= ((valid >> u) & 1u) && sub == (uint32_t)s2.bin ? (1u << u) : 0u;
    }
    // both counts are at most kLdsCand: one packed 16+16-bit prefix sum
    uint32_t tot;
    const uint32_t before = block_exclusive_scan(__popc(hi) | (__popc(eq) << 16), lds.scratch, tot);
    const uint32_t n_surv = s2.count, R2 = R - s2.above;
    // Survivors go to the end of lds.cand; the staged positions fill words
    // 0..s2.above-1 of hist + cand, below them (s2.above + n_surv <= in_bin).
    cbase = kLdsCand - (int)n_surv;
    uint32_t* stage = reinterpret_cast<uint32_t*>(&lds);
    const bool staged = a.out_scores == nullptr;
    uint32_t slot = before & 0xFFFFu, cs = (uint32_t)cbase + (before >> 16);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (hi & (1u << u)) {
        if (staged) {
          stage[slot] = jx[u];
        } else {
          put_selection(a, above + slot, (int)jx[u], score_of(kx[u], bx[u], (int)jx[u]));
        }
        ++slot;
      }
      if (eq & (1u << u)) lds.cand[cs++] = make_uint2(bx[u], jx[u]);
    }
    if (tid == 0) lds.cnt = above + s2.above;
    __syncthreads();
    if (staged) {
      for (uint32_t q = tid; q < s2.above; q += kBlock) put_selection(a, above + q, (int)stage[q], 0.f);
    }
    if (n_surv <= (uint32_t)kBlock) {
      if (tid < (int)n_surv) {
        const uint2 me = lds.cand[cbase + tid];
        const uint32_t mk = src == kSrcLds ? me.x : score_key(__uint_as_float(me.x));
        uint32_t rank = 0;
        for (uint32_t o = 0; o < n_surv; ++o) {
          const uint2 c = lds.cand[cbase + o];
          const uint32_t ok = src == kSrcLds ? c.x : score_key(__uint_as_float(c.x));
          rank += (ok > mk || (ok == mk && c.y < me.y)) ? 1u : 0u;
        }
        if (rank < R2) put_selection(a, above + s2.above + rank, (int)me.y, score_of(mk, me.x, (int)me.y));
      }
      return;
    }
    n_src = (int)n_surv;  // the last pass reads the compacted sub-bin
  } else {
    for (int x = tid; x < kHistBins; x += kBlock) lds.hist[x] = 0u;
    __syncthreads();
    for (int e = tid; e < n_src; e += kBlock) {
      uint32_t key;
      int j;
      if (fetch(e, key, j)) atomicAdd(&lds.hist[(key >> 10) & 0x7FFu], 1u);
    }
    __syncthreads();
    s2 = find_bin_of_rank(lds.hist, kHistBins, R, lds.scratch);
    for (int e = tid; e < n_src; e += kBlock) {
      uint32_t key;
      int j;
      if (fetch(e, key, j) && ((key >> 10) & 0x7FFu) > (uint32_t)s2.bin) emit(j);
    }
  }
  const uint32_t R2 = R - s2.above;
  const uint32_t pre2 = (B1 << 11) | (uint32_t)s2.bin;  // key >> 10 of the survivors

  // pass 3: key bits 9..0
  __syncthreads();
  for (int x = tid; x < 1024; x += kBlock) lds.hist[x] = 0u;
  __syncthreads();
  for (int e = tid; e < n_src; e += kBlock) {
    uint32_t key;
    int j;
    if (fetch(e, key, j) && (key >> 10) == pre2) atomicAdd(&lds.hist[key & 0x3FFu], 1u);
  }
  __syncthreads();
  const BinSplit s3 = find_bin_of_rank(lds.hist, 1024, R2, lds.scratch);
  const uint32_t kstar = (pre2 << 10) | (uint32_t)s3.bin;
  for (int e = tid; e < n_src; e += kBlock) {
    uint32_t key;
    int j;
    if (fetch(e, key, j) && (key >> 10) == pre2 && (key & 0x3FFu) > (uint32_t)s3.bin) emit(j);
  }
  const uint32_t R3 = R2 - s3.above;  // tokens to take among those with key == kstar

  if (s3.count == R3) {
    for (int e = tid; e < n_src; e += kBlock) {
      uint32_t key;
      int j;
      if (fetch(e, key, j) && key == kstar) emit(j);
    }
  } else {
    // More exact ties than places: take the lowest token indices, scanning
    // the scores in index order.
    __syncthreads();
    uint32_t taken = 0;
    for (int jb = 0; jb < n_valid && taken < R3; jb += kBlock) {
      const int j = jb + tid;
      const bool f = j < n_valid && score_key(load_coherent(a.scores + j)) == kstar;
      uint32_t tot;
      const uint32_t before = block_exclusive_scan(f ? 1u : 0u, lds.scratch, tot);
      if (f && taken + before < R3) emit(j);
      taken += tot;
    }
  }
}

// The remaining tokens of bin B1, once every slice is done.  Leaves the
// histogram row zero.  With `have_known`, `known` is the histogram split a
// slice of this workgroup already found (the histogram is final before any
// slice runs); otherwise the histogram is read again.  on_final(n) is called by every
// thread as soon as the output slots 0..n-1 are final (the tokens above bin
// B1, which the slices wrote, or all k slots when every valid token is
// selected), while the candidates are still loading.
template <class OnFinal>
__device__ __forceinline__ void resolve_query(const SelectArgs& a, ResolveLds& lds, bool have_known, BinSplit known,
                                              OnFinal on_final) {
  const int tid = thread_index();
  // The first kLdsCand candidates are requested first (entries past the
  // list's count are never used).
  constexpr int kPer = kLdsCand / kBlock;
  uint64_t c[kPer];
  const bool resolve = a.n_valid > a.k;
  if (resolve) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) c[u] = load_coherent(a.cand + u * kBlock + tid);
  }
  const BinSplit sp = have_known ? known : kth_bin(a, lds.scratch);
  on_final(resolve ? sp.above : (uint32_t)a.k);
  for (int x = tid; x < kHistBins; x += kBlock) a.ghist[x] = 0u;
  if (!resolve) return;  // the filter items wrote everything
  const uint32_t in_bin = sp.count;
  const bool use_cand = in_bin <= (uint32_t)kCandCap;
  const bool in_lds = in_bin <= (uint32_t)kLdsCand;
  if (in_lds) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) lds.cand[u * kBlock + tid] = make_uint2((uint32_t)c[u], (uint32_t)(c[u] >> 32));
  }
  pick_in_bin(a, lds, (uint32_t)sp.bin, sp.above, in_bin, in_lds ? kSrcLds : (use_cand ? kSrcList : kSrcScores));
}

// ---------------------------------------------------------------------------
// select_query: the whole top-k of one query token in one workgroup, for
// score rows of at most kSelectMax: the histogram gives bin B1 of the k-th
// largest score, one streaming pass over the scores marks the tokens of
// higher bins and collects bin B1's tokens in LDS, then the marked tokens
// are written and pick_in_bin takes the rest.  Leaves the histogram row zero.
// ---------------------------------------------------------------------------
constexpr int kSelPer = 16;            // scores per thread per batch
constexpr int kSelBatch = kBlock * kSelPer;
static_assert(kSelectMax / kSelBatch == kSelBatchesMax, "select batches");
constexpr int kSelAhead = 3;           // batches in flight beyond the one being classified

__device__ __forceinline__ void select_query(const SelectArgs& a, ResolveLds& lds) {
  const int tid = thread_index();
  const int n_valid = a.n_valid, k = a.k;
  if (n_valid <= k) {  // at most k valid tokens: all of them, then -1 padding
    for (int x = tid; x < kHistBins; x += kBlock) a.ghist[x] = 0u;
    for (int j = tid; j < k; j += kBlock) {
      if (j < n_valid) {
        put_selection(a, (uint32_t)j, j, a.out_scores ? load_coherent(a.scores + j) : 0.f);
      } else {
        store_coherent(reinterpret_cast<uint32_t*>(a.out + j), 0xffffffffu);
        if (a.out_scores) store_coherent(a.out_scores + j, __uint_as_float(0x7fc00000u));
      }
    }
    return;
  }
  // Each score line was written whole by one scan workgroup earlier in this
  // launch and is not cached on this die before, so plain 16-byte loads
  // read it current.  The loop issues no store and no barrier, so the loads
  // of kSelAhead batches stay in flight while one is classified; the first
  // ones are issued before the histogram is read.
  // Loads are unconditional (past the valid scores they all read the row's
  // last valid 64 bytes, one cache line) so the compiler can count the
  // outstanding loads exactly and keep kSelAhead batches in flight.
  const int last = ((n_valid + kSelPer - 1) & ~(kSelPer - 1)) - kSelPer;
  auto load_batch = [&](f32x4_t* v, int b) {
    const int j0 = min(b * kSelBatch + tid * kSelPer, last);
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(a.scores + j0);
#pragma unroll
    for (int q = 0; q < kSelPer / 4; ++q) v[q] = src[q];
  };
  f32x4_t v[kSelAhead + 1][kSelPer / 4];
#pragma unroll
  for (int b = 0; b < kSelAhead; ++b) load_batch(v[b], b);
  if (tid == 0) lds.cnt = 0u;  // candidate count while streaming
  const BinSplit sp = kth_bin(a, lds.scratch);
  for (int x = tid; x < kHistBins; x += kBlock) a.ghist[x] = 0u;
  const uint32_t B1 = (uint32_t)sp.bin, above = sp.above, in_bin = sp.count;
  const bool in_lds = in_bin <= (uint32_t)kLdsCand;
  const int nb = (n_valid + kSelBatch - 1) / kSelBatch;

  // Bit u of lds.marks[b][tid]: token b * kSelBatch + tid * kSelPer + u is
  // above B1.  The batch loop is rolled over groups of kSelAhead + 1 batches
  // (a static ring of registers within a group).
  // The bin tests as two float comparisons against the smallest values of
  // bins B1 and B1 + 1: key order is float order except that -0 and +0
  // have different keys, NaN has key 0, and the keys of bins 0..3 below
  // -inf's are NaN bit patterns.  So the integer keys decide when a bound
  // is +0 (B1 is 1023 or 1024), when B1 is below bin 4, or when B1 + 1
  // would be past +inf's bin.
  const bool fcmp = B1 >= 4u && B1 != 1023u && B1 != 1024u && B1 <= 2043u;
  const float f_lo = key_value(B1 << kHistShift), f_hi = key_value((B1 + 1u) << kHistShift);
  uint32_t mine = 0;
  for (int b0 = 0; b0 < nb; b0 += kSelAhead + 1) {
#pragma unroll
    for (int bb = 0; bb <= kSelAhead; ++bb) {
      const int b = b0 + bb;
      load_batch(v[(bb + kSelAhead) % (kSelAhead + 1)], b + kSelAhead);
      if (b >= nb) continue;  // uniform
      const f32x4_t* cur = v[bb];
      const int j0 = b * kSelBatch + tid * kSelPer;
      const int n_in = max(0, min(kSelPer, n_valid - j0));
      const uint32_t in_mask = n_in >= 32 ? 0xFFFFFFFFu : ((1u << n_in) - 1u);
      uint32_t hi = 0, eq = 0;
      if (fcmp) {
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
          const float x = cur[u >> 2][u & 3];
          const bool above_hi = x >= f_hi;
          hi |= above_hi ? (1u << u) : 0u;
          eq |= (!above_hi && x >= f_lo) ? (1u << u) : 0u;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
          const uint32_t bin = score_key(cur[u >> 2][u & 3]) >> kHistShift;
          hi |= bin > B1 ? (1u << u) : 0u;
          eq |= bin == B1 ? (1u << u) : 0u;
        }
      }
      hi &= in_mask;
      eq &= in_mask;
      lds.marks[b][tid] = (uint16_t)hi;
      mine += __popc(hi);
      // Candidates go to LDS now (an LDS atomic, no memory wait), without
      // branches: lanes write every slot u, the ones that are not
      // candidates into a spare entry.  They hold the score bits; the radix
      // passes turn the few real candidates into keys.
      if (in_lds && __ballot(eq != 0u) != 0ull) {
        uint32_t c = 0;
        if (eq) c = atomicAdd(&lds.cnt, (uint32_t)__popc(eq));
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
          const uint32_t pos = ((eq >> u) & 1u) ? c + (uint32_t)__popc(eq & ((1u << u) - 1u)) : (uint32_t)kLdsCand;
          lds.cand[min(pos, (uint32_t)kLdsCand)] = make_uint2(__float_as_uint(cur[u >> 2][u & 3]), (uint32_t)(j0 + u));
        }
      }
    }
  }
  // The marked tokens take slots 0..above-1.
  uint32_t n_hi;
  uint32_t slot = block_exclusive_scan(mine, lds.scratch, n_hi);
  const uint32_t n_cand = lds.cnt;
  // Two copies of the write loop: without the score output it holds no load,
  // so its stores need not wait for one another.
  auto write_marked = [&](auto with_scores) {
    for (int b = 0; b < nb; ++b) {
      uint32_t bits = lds.marks[b][tid];
      while (bits) {
        const int u = __builtin_ctz(bits);
        bits &= bits - 1u;
        const int j = b * kSelBatch + tid * kSelPer + u;
        put_selection(a, slot++, j, with_scores ? load_coherent(a.scores + j) : 0.f);
      }
    }
  };
  if (!a.out_scores && n_hi <= (uint32_t)kHistBins) {
    // Positions staged in the histogram's LDS (free until pick_in_bin),
    // then written to consecutive slots by consecutive lanes.
    for (int b = 0; b < nb; ++b) {
      uint32_t bits = lds.marks[b][tid];
      while (bits) {
        const int u = __builtin_ctz(bits);
        bits &= bits - 1u;
        lds.hist[slot++] = (uint32_t)(b * kSelBatch + tid * kSelPer + u);
      }
    }
    __syncthreads();
    for (uint32_t q = tid; q < n_hi; q += kBlock) put_selection(a, q, (int)lds.hist[q], 0.f);
  } else if (a.out_scores) {
    write_marked(std::true_type{});
  } else {
    write_marked(std::false_type{});
  }
  if (n_hi != above || (in_lds && n_cand != in_bin)) {  // never expected: counts disagree with the histogram
    if (tid == 0) raise_error(a.err, kErrSelection);
    return;
  }
  pick_in_bin(a, lds, B1, above, in_bin, in_lds ? kSrcLdsBits : kSrcScores);
}

}  // namespace mono
