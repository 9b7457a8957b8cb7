// Host-side plan of libmono_decode.so, in plain C++ (no HIP): the shape
// constants of the kernels, the argument checks of every C-ABI call, the
// workspace layout of the step kernel and the launch plan (how work is cut
// into items and which kernel instance runs).  The library compiles it with
// its kernels; a host test compiles it alone with g++ under the address and
// undefined-behaviour sanitizers and drives every check through it.
//
// Geometry (page "vllm.models.minimax_m3.amd.ops.mxfp4_pages", module
// docstring): a page is 128 token rows of 64 packed e2m1 bytes, then 128
// rows of 4 e8m0 scale bytes, 8704 B.  Step tables (page
// "vllm.models.minimax_m3.amd.mono.dispatch", _step_refusal): one int32
// block table with rows bt_stride apart, int32 seq_lens, T tokens decoded
// per request.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mono_decode.h"

namespace mono {

// ---- shapes ------------------------------------------------------------------
constexpr int kBlock = 256;  // threads of every workgroup (4 x wave64)
constexpr int kWaves = kBlock / 64;
constexpr int kPageTokens = 128;
constexpr int kHeadDim = 128;
constexpr int kQHeads = 16;  // query heads per KV head
constexpr int kMaxBtStride = 1 << 20;  // 2^27 tokens per request
constexpr int kMaxHeads = 64;
constexpr int kMergeMaxCandidates = 8192;  // topk merge: G * k_in per query token

// Scan and selection items (topk_device.h).
constexpr int kScanChunkPages = 16;  // index pages per scan work item (default)
constexpr int kMaxChunkPages = 64;   // one page id per lane of a wave
// The largest scan chunk the plan makes.  With ragged lengths the chunks
// that hold pages do not divide into whole rounds of the workgroups, and
// the last round's chunks set the end of the scan: 32-page chunks measured
// faster than 64 on a batch of 16K-64K contexts (16-page ones slower: each
// chunk flushes its histograms and arrives once).
constexpr int kPlanChunkPages = 32;
constexpr int kHistBins = 2048;      // top 11 bits of the score key
constexpr int kHistShift = 21;
constexpr int kSlice = 4096;         // scores per filter work item
constexpr int kCandCap = 8192;       // candidates kept per query token
constexpr int kSelectMax = 65536;    // longest score row a single workgroup selects from

// Step kernel (step.hip).
constexpr size_t kClearBytes = 32768;  // bytes zeroed by one clear item
constexpr int kMinSplitTokens = 256;   // attention candidates per split: one pass of 4 waves x 4 groups of 16
constexpr int kMaxSplitTokens = 8192;
constexpr int kFusedAttnRounds = 2;   // attention splits of the one-launch step: up to 2 rounds of workgroups
// Chunk-local step: scores a scan item keeps in LDS (32 pages), and chunks
// per request (its attention splits).
constexpr int kLocalTokens = 4096;
constexpr int kLocalMaxChunks = 16;
constexpr int kLvlWords = 5;     // per query token: arrivals of the four levels, then the finished count
constexpr int kExchCap = 2048;   // threshold-bin tokens a request's chunks exchange (more: radix levels)

enum StepMode { kModeIndex = 1, kModeAttn = 2, kModeFused = 3 };
enum CacheFormat { kFmtMxfp4 = 0, kFmtFp8 = 1 };

// Header words of the control block (the same offset in every layout).
constexpr uint32_t kHdrTicket = 0;   // next work-item ticket
constexpr uint32_t kHdrExits = 1;    // workgroups that have left
constexpr uint32_t kHdrCleared = 2;  // clear items done
constexpr uint32_t kHdrZeroed = 3;   // zero region the last call left clean, in 256-B units
constexpr uint32_t kHdrWords = 4;
// Work-item descriptors: kind in the top bits, index below.
// kItemAttnGated: an attention split published before its row's selection
// is complete, which waits for the row's ready word before reading it.
constexpr uint32_t kItemScan = 1, kItemFilter = 2, kItemAttn = 3, kItemSelect = 4, kItemAttnGated = 5;
constexpr uint32_t kKindShift = 28;
constexpr uint32_t kIndexMask = (1u << kKindShift) - 1u;

struct StepLayout {
  int mode, B, T, H, k, sparse;
  int G;             // index-q heads scored per query token (index call only; else 1)
  // Index rows: G * B * T, row (h, b, t) at h * B * T + b * T + t.  A
  // request's rows are its G * T (head, token) pairs u = h * T + t.
  int q_groups;      // ceil(G * T / 4) row groups per request
  int chunk_pages;   // index pages per scan chunk
  int chunks;        // scan chunks per query group (window pages / chunk_pages, rounded up)
  int win_lo, win_hi;  // page window [win_lo, win_hi) of every request the index items score
  int lcap;          // bt_stride * 128: capacity of a score row
  int slices;        // filter slices per query token (lcap / 4096, rounded up)
  int split_tokens;  // attention candidates per split
  int n_splits;      // attention splits per (query token, KV head)
  int select_mode;   // 1: one workgroup selects each query token's top k
  int local;         // 1: chunk-local step (one query token per request; see step.hip)
  int local_filter;  // 1: each scan chunk filters its own scores as a slice of its row (see scan_item)
  int part_splits;   // splits the partial buffers hold per (query token, KV head)
  uint32_t n_clear, n_scan, n_select, n_filter, n_attn;  // work items of each kind (clear: when needed)
  uint32_t n_ready0;    // items ready at the start (the first tickets after the clear items)
  uint32_t ready_kind;  // their kind
  uint32_t n_queue;     // items published into the ready queue while the kernel runs
  size_t zero_end;      // [ctrl_base + header, zero_end) must be zero when items start
  uint64_t zero_units;  // zero_end / 256
  // control block (u32 words from ctrl_base): word offsets
  size_t ctrl, scan_done, filter_cnt, out_cnt, cand_cnt, attn_cnt, sel_ready, lvl_cnt, pub, queue, ctrl_words;
  int has_sel_ready;  // one-launch step: a ready word per (row, KV head): the row's selection is complete
  // byte offsets in the workspace (hist2, hist3, ties, xcand, xcnt: chunk-local step only)
  size_t err, ctrl_base, hist, hist2, hist3, ties, scores, xcand, xcnt, cand, pm, pl, pacc, total;
};

// Workspace layout of one call (mode, shapes); sizes only, no device state.
// G > 1 only for the index call (mode kModeIndex).
StepLayout step_layout(int mode, int B, int T, int H, int bt_stride, int k, int sparse, int G = 1);

// Kernel instances of the step kernel: [1, 4 query tokens] x [MXFP4, fp8],
// then the chunk-local instances [MXFP4, fp8], then the attention-only
// instances [MXFP4, fp8] (the attention call's items alone).
constexpr int kStepVariants = 8;
inline int step_variant(bool tq4, bool fp8) { return (tq4 ? 1 : 0) + (fp8 ? 2 : 0); }
inline int local_variant(bool fp8) { return fp8 ? 5 : 4; }
inline int attn_variant(bool fp8) { return fp8 ? 7 : 6; }

// What the device offers: compute units and, per kernel instance, how many
// workgroups fit at once (occupancy x compute units).
struct DeviceShape {
  int cus;
  int resident[kStepVariants];
};

// Cuts a call's work into items for the device: scan chunk sizes, the
// selection mode, attention split sizes and, for the one-launch call with
// one query token per request, whether the chunk-local instance runs.  The
// chunk-local instance is chosen only when every chunk item is a first-round
// item of a grid that fits on the device at once (its chunks wait for each
// other).  Returns the grid (0: nothing to do) or a negative MONO_E* code;
// *variant receives the kernel instance.
long plan_step(StepLayout& lay, const DeviceShape& dev, bool fp8, bool has_sel_scores, int* variant,
               const char* what);

// ---- errors --------------------------------------------------------------------
// Records a formatted message as the calling thread's last error; returns `code`.
int set_error(int code, const char* fmt, ...);
void clear_error();
const char* last_error();

// ---- argument checks of the C-ABI calls (no device access) ---------------------
int check_step_shape(int B, int T, int bt_stride, int k, bool need_k);
int check_pages_args(const void* a, const void* b, const void* c, int64_t n_pages, size_t align_a, size_t align_b,
                     size_t align_c, const char* what);
int check_index_call(const char* what, const void* index_q, const void* index_pages, int64_t num_pages,
                     const void* block_table, int bt_stride, const void* seq_lens, int B, int T, int k,
                     const void* selected_idx, const void* selected_scores, const void* ws, size_t ws_bytes,
                     int page_lo, int page_hi, StepLayout* lay);
int check_pa_call(const char* what, const void* q, const void* k_pages, const void* v_pages, int64_t num_pages,
                  int kv_heads, const void* block_table, int bt_stride, const void* seq_lens, int B, int T,
                  const void* selected_idx, int k, float scale, float k_scale, float v_scale, const void* out,
                  const void* ws, size_t ws_bytes, StepLayout* lay);
// ws == nullptr with ws_bytes == SIZE_MAX: the caller's static scratch (checked by the caller).
int check_sparse_call(const char* what, const void* index_q, const void* index_pages, const void* q,
                      const void* k_pages, const void* v_pages, int64_t num_pages, int kv_heads,
                      const void* block_table, int bt_stride, const void* seq_lens, int B, int T, int k,
                      float scale, float k_scale, float v_scale, const void* selected_idx, const void* out,
                      const void* ws, size_t ws_bytes, StepLayout* lay);
int check_merge_call(const void* cand_idx, const void* cand_scores, int G, int64_t N, int k_in, int k_out,
                     const void* out_idx, const void* out_scores);
// Indexer context parallelism on one device: the index layout of G heads
// (its workspace first) and the shard candidate buffers after it.
struct CpLayout {
  StepLayout index;    // the index call over G heads, one page window at a time
  int shards;          // shards with a non-empty window (windows past the table are empty)
  int width;           // block-table columns per shard window: ceil(bt_stride / shards)
  size_t cand_idx;     // byte offset of int32 [shards, G*B*T, k] candidate positions
  size_t cand_scores;  // byte offset of fp32 [shards, G*B*T, k] candidate scores
  size_t total;
};
CpLayout cp_layout(int B, int T, int G, int bt_stride, int k, int shards);
int check_cp_call(const void* index_q, const void* index_pages, int64_t num_pages, const void* block_table,
                  int bt_stride, const void* seq_lens, int B, int T, int G, int k, int shards, const void* out,
                  const void* ws, size_t ws_bytes, CpLayout* lay);
int check_insert_call(const void* k_rows, const void* v_rows, const void* index_rows, const void* slots, int64_t n,
                      int kv_heads, const void* k_pages, const void* v_pages, const void* index_pages,
                      int64_t num_pages, const void* err);
int check_bench_read_call(const void* pages, const void* page_ids, int64_t n_pages, int mode, int grid,
                          const void* sink);
int check_bench_scan_call(const void* index_q, const void* pages, int64_t num_pages, const void* block_table,
                          int bt_stride, const void* seq_lens, int B, int chunk_pages, int variant, const void* hist,
                          const void* err);

}  // namespace mono
