// Host-side plan of libmono_decode.so in plain C++ (see plan.h): argument
// checks, the step kernel's workspace layout and its launch plan.
#include "plan.h"

#include <stdarg.h>
#include <stdio.h>

#include <algorithm>

namespace mono {

// ---- errors --------------------------------------------------------------------
namespace {
thread_local char g_error[512] = "";

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool finite(float x) { return x == x && x != __builtin_inff() && x != -__builtin_inff(); }
// fp8 tensor scales must be finite and positive.
bool bad_tensor_scale(float x) { return !(x > 0.f) || x == __builtin_inff(); }
}  // namespace

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_error[0] = '\0'; }

const char* last_error() { return g_error; }

// ---- workspace layout ------------------------------------------------------------
StepLayout step_layout(int mode, int B, int T, int H, int bt_stride, int k, int sparse, int G) {
  StepLayout l{};
  l.mode = mode;
  l.B = B;
  l.T = T;
  l.H = H;
  l.k = k;
  l.sparse = sparse;
  l.G = G;
  const size_t N = (size_t)G * B * T;  // index rows (query tokens when G == 1)
  l.q_groups = (G * T + 3) / 4;
  l.chunk_pages = kScanChunkPages;  // plan_step re-balances this to the resident workgroups
  l.chunks = (bt_stride + l.chunk_pages - 1) / l.chunk_pages;
  l.lcap = bt_stride * kPageTokens;
  l.win_lo = 0;  // the index call over a page window narrows these
  l.win_hi = bt_stride;
  l.slices = (l.lcap + kSlice - 1) / kSlice;
  const bool index = (mode & kModeIndex) != 0, attn = (mode & kModeAttn) != 0;
  // Attention splits: 256 candidates per workgroup unless that makes more
  // than 4096 items (plan_step may enlarge them; the partial buffers are
  // sized for this count).
  const long list_max = sparse ? (long)k : (long)l.lcap;
  const size_t NH = N * H;
  int split = kMinSplitTokens;
  while (split < kMaxSplitTokens && NH * (size_t)((list_max + split - 1) / split) > 4096) split *= 2;
  l.split_tokens = split;
  l.n_splits = (int)((list_max + split - 1) / split);

  // Selection by slices and a resolve; plan_step may switch to one
  // workgroup per query token instead (the queue is sized for slices, the
  // larger of the two).
  l.select_mode = 0;
  l.local = 0;  // plan_step decides
  // The one-launch step with one query token per request may run chunk-local
  // (plan_step decides); it needs room for up to kLocalMaxChunks splits.
  const bool local_ok = mode == kModeFused && T == 1;
  l.n_scan = index ? (uint32_t)(B * l.q_groups * l.chunks) : 0u;
  l.n_select = 0u;
  l.n_filter = index ? (uint32_t)(N * l.slices) : 0u;
  l.n_attn = attn ? (uint32_t)(NH * l.n_splits) : 0u;
  // Items ready at the start take the first tickets; the rest are published.
  l.n_ready0 = index ? l.n_scan : l.n_attn;
  l.ready_kind = index ? kItemScan : kItemAttn;
  l.n_queue = index ? l.n_select + l.n_filter + l.n_attn : 0u;

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  l.err = take(256);
  // Control block: u32 words zeroed by the last workgroup of every call.
  // Its 4-word header sits at the same offset in every layout.
  size_t w = 0;
  l.ctrl = w;
  w += kHdrWords;
  l.scan_done = w;
  w += index ? (size_t)B * l.q_groups : 0;
  l.filter_cnt = w;
  w += index ? N : 0;
  l.out_cnt = w;
  w += index ? N : 0;
  l.cand_cnt = w;
  w += index ? N : 0;
  l.attn_cnt = w;
  w += attn ? NH : 0;
  l.sel_ready = w;
  l.has_sel_ready = index && attn;
  w += l.has_sel_ready ? NH : 0;
  l.lvl_cnt = w;
  w += local_ok ? N * kLvlWords : 0;
  l.pub = w;
  w += 1;
  l.queue = w;
  w += l.n_queue;
  l.ctrl_words = w;
  l.ctrl_base = take(w * 4);
  l.hist = take(index ? N * kHistBins * 4 : 0);
  l.hist2 = take(local_ok ? N * kHistBins * 4 : 0);
  l.hist3 = take(local_ok ? N * 1024 * 4 : 0);
  l.ties = take(local_ok ? N * kLocalMaxChunks * 4 : 0);
  l.xcand = take(local_ok ? N * kLocalMaxChunks * (size_t)kExchCap * 8 : 0);
  l.xcnt = take(local_ok ? N * kLocalMaxChunks * 4 : 0);
  // Everything from the end of the header to here must be zero when the
  // items start; the rest is scratch that each call overwrites.
  l.zero_end = off;
  l.zero_units = (uint64_t)(off >> 8);
  const size_t zero_bytes = off - (l.ctrl_base + kHdrWords * 4);
  l.n_clear = (uint32_t)((zero_bytes + kClearBytes - 1) / kClearBytes);
  l.scores = take(index ? N * (size_t)l.lcap * 4 : 0);
  l.cand = take(index ? N * (size_t)kCandCap * 8 : 0);
  l.part_splits = local_ok ? std::max(l.n_splits, kLocalMaxChunks) : l.n_splits;
  const size_t S = (size_t)l.part_splits;
  l.pm = take(attn ? NH * S * kQHeads * 4 : 0);
  l.pl = take(attn ? NH * S * kQHeads * 4 : 0);
  l.pacc = take(attn ? NH * S * kQHeads * kHeadDim * 4 : 0);
  l.total = off;
  return l;
}

// ---- launch plan -------------------------------------------------------------------
long plan_step(StepLayout& lay, const DeviceShape& dev, bool fp8, bool has_sel_scores, int* variant,
               const char* what) {
  const bool tq4 = lay.G * lay.T > 1 && (lay.mode & kModeIndex);
  *variant = step_variant(tq4, fp8);
  if (lay.mode == kModeAttn && dev.resident[attn_variant(fp8)] > 0) *variant = attn_variant(fp8);
  int cap = std::max(1, dev.resident[*variant]);
  if (lay.mode & kModeIndex) {
    // Scan chunks sized so the scan items make about one round of the
    // resident workgroups (all of them start together and end together).
    const int groups = lay.B * lay.q_groups;
    const int span = lay.win_hi - lay.win_lo;  // pages of the window (the whole table by default)
    const int per_group = std::max(1, cap / std::max(1, groups));
    lay.chunk_pages = std::min(kPlanChunkPages, std::max(1, (span + per_group - 1) / per_group));
    lay.chunks = (span + lay.chunk_pages - 1) / lay.chunk_pages;
    lay.n_scan = (uint32_t)((size_t)groups * lay.chunks);
    lay.n_ready0 = lay.n_scan;
    // Rows of at most kSelectMax scores are selected by one workgroup each
    // (inline in the last scan chunk when a request has one query token)
    // once the slices would take more than two rounds of the resident
    // workgroups; with fewer query tokens, slices spread each selection
    // over more compute units and finish sooner.
    const size_t N = (size_t)lay.G * lay.B * lay.T;
    if ((size_t)span * kPageTokens <= kSelectMax && N * (size_t)lay.slices > 2 * (size_t)cap) {
      lay.select_mode = 1;
      lay.n_filter = 0u;
      lay.n_select = lay.G * lay.T > 1 ? (uint32_t)N : 0u;
      lay.n_queue = lay.n_select + lay.n_attn;
    }
  }
  if (lay.mode & kModeAttn) {
    // Attention splits as large as it takes to make about one round of the
    // resident workgroups (never smaller than the layout's, whose partial
    // buffers are sized for the most splits).  In the one-launch step the
    // splits are published as selections finish, so two rounds' worth lets
    // the workgroups that are free by then share the last tokens' attention.
    const size_t NH = (size_t)lay.B * lay.T * lay.H;
    const long list_max = lay.sparse ? (long)lay.k : (long)lay.lcap;
    int split = lay.split_tokens;
    const size_t acap = (size_t)cap * (lay.mode == kModeFused ? kFusedAttnRounds : 1);
    while (split < kMaxSplitTokens && NH * (size_t)((list_max + split - 1) / split) > acap) split *= 2;
    lay.split_tokens = split;
    lay.n_splits = (int)((list_max + split - 1) / split);
    lay.n_attn = (uint32_t)(NH * lay.n_splits);
    if (!(lay.mode & kModeIndex)) lay.n_ready0 = lay.n_attn;
    lay.n_queue = (lay.mode & kModeIndex) ? lay.n_select + lay.n_filter + lay.n_attn : 0u;
  }
  if (lay.mode == kModeFused && lay.T == 1 && lay.part_splits >= kLocalMaxChunks && !has_sel_scores &&
      lay.win_lo == 0) {
    // Chunk-local step: at most kLocalMaxChunks chunks of at most
    // kLocalTokens scores per request, and every scan item a first ticket
    // of a resident workgroup of its own kernel instance (the chunks of a
    // request wait for each other).  Otherwise the item-queue instance runs.
    const int lvariant = local_variant(fp8);
    const int lcap = dev.resident[lvariant];
    const int groups = lay.B;
    const int span = lay.win_hi - lay.win_lo;
    const int per_group = std::max(1, lcap / std::max(1, groups));
    const int cp = std::max((span + per_group - 1) / per_group, (span + kLocalMaxChunks - 1) / kLocalMaxChunks);
    const int ch = (span + cp - 1) / cp;
    if (lcap > 0 && cp * kPageTokens <= kLocalTokens && ch <= kLocalMaxChunks &&
        (size_t)groups * ch <= (size_t)lcap) {
      *variant = lvariant;
      cap = lcap;
      lay.local = 1;
      lay.chunk_pages = cp;
      lay.chunks = ch;
      lay.n_scan = (uint32_t)(groups * ch);
      lay.n_ready0 = lay.n_scan;
      lay.select_mode = 0;
      lay.n_select = lay.n_filter = lay.n_attn = 0u;
      lay.n_queue = 0u;
    }
  }
  if (!lay.local && (lay.mode & kModeIndex) && lay.G == 1 && lay.T == 1 && !lay.select_mode && !has_sel_scores &&
      lay.win_lo == 0 && lay.chunk_pages * kPageTokens <= kSlice && lay.n_scan <= (uint32_t)cap) {
    // Local filtering: every scan chunk is a first-round ticket of the
    // resident workgroups (the chunks of a row wait for the row's
    // histogram), and a chunk's scores fit one slice.
    lay.local_filter = 1;
    lay.n_filter = 0u;
    lay.n_queue = lay.n_select + lay.n_filter + lay.n_attn;
  }
  const uint64_t n_items = (uint64_t)lay.n_clear + lay.n_ready0 + lay.n_queue;
  if (n_items == 0) return 0;
  if ((uint64_t)lay.n_scan + lay.n_select + lay.n_filter + lay.n_attn > kIndexMask)
    return set_error(MONO_ENOTSUP, "%s: too many work items", what);
  if (lay.zero_units > 0xFFFFFFFFull || lay.ctrl_base != 256)
    return set_error(MONO_ENOTSUP, "%s: workspace layout too large", what);
  return (long)std::min<uint64_t>(n_items, (uint64_t)cap);
}

// ---- argument checks ---------------------------------------------------------------
int check_step_shape(int B, int T, int bt_stride, int k, bool need_k) {
  if (B < 1) return set_error(MONO_EINVAL, "B must be >= 1 (got %d)", B);
  if (T < 1) return set_error(MONO_EINVAL, "T must be >= 1 (got %d)", T);
  if ((long long)B * T > (1LL << 30)) return set_error(MONO_EINVAL, "B*T too large (%d x %d)", B, T);
  if (bt_stride < 1 || bt_stride > kMaxBtStride)
    return set_error(MONO_EINVAL, "bt_stride must be in [1, %d] (got %d)", kMaxBtStride, bt_stride);
  if (need_k && k < 1) return set_error(MONO_EINVAL, "k must be >= 1 (got %d)", k);
  if (need_k && k > bt_stride * MONO_PAGE_TOKENS)
    return set_error(MONO_EINVAL, "k (%d) exceeds the block table's capacity (%d tokens)", k,
                     bt_stride * MONO_PAGE_TOKENS);
  return MONO_OK;
}

int check_pages_args(const void* a, const void* b, const void* c, int64_t n_pages, size_t align_a, size_t align_b,
                     size_t align_c, const char* what) {
  if (n_pages < 0) return set_error(MONO_EINVAL, "%s: n_pages < 0", what);
  if (n_pages > (int64_t)1 << 34) return set_error(MONO_EINVAL, "%s: n_pages too large", what);
  if (n_pages == 0) return MONO_OK;
  if (!a || !b || !c) return set_error(MONO_EINVAL, "%s: NULL buffer", what);
  if (!aligned(a, align_a) || !aligned(b, align_b) || !aligned(c, align_c))
    return set_error(MONO_EINVAL, "%s: buffers need %zu-, %zu- and %zu-byte alignment", what, align_a, align_b,
                     align_c);
  return MONO_OK;
}

int check_index_call(const char* what, const void* index_q, const void* index_pages, int64_t num_pages,
                     const void* block_table, int bt_stride, const void* seq_lens, int B, int T, int k,
                     const void* selected_idx, const void* selected_scores, const void* ws, size_t ws_bytes,
                     int page_lo, int page_hi, StepLayout* lay) {
  if (int rc = check_step_shape(B, T, bt_stride, k, true)) return rc;
  if (page_hi < 0) page_hi = bt_stride;
  if (page_lo < 0 || page_lo >= page_hi || page_hi > bt_stride)
    return set_error(MONO_EINVAL, "%s: page window [%d, %d) not inside [0, %d)", what, page_lo, page_hi, bt_stride);
  if (!index_q || !index_pages || !block_table || !seq_lens || !selected_idx || !ws)
    return set_error(MONO_EINVAL, "%s: NULL buffer", what);
  if (num_pages < 1) return set_error(MONO_EINVAL, "%s: num_pages must be >= 1", what);
  if (!aligned(index_q, 16) || !aligned(index_pages, 16) || !aligned(ws, 256) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(selected_idx, 4) || !aligned(selected_scores, 4))
    return set_error(MONO_EINVAL, "%s: index_q/pages need 16-byte, ws 256-byte, tables 4-byte alignment", what);
  *lay = step_layout(kModeIndex, B, T, 1, bt_stride, k, 1);
  if (ws_bytes < lay->total) return set_error(MONO_ENOSPC, "%s: workspace %zu B < %zu B", what, ws_bytes, lay->total);
  lay->win_lo = page_lo;
  lay->win_hi = page_hi;
  return MONO_OK;
}

int check_pa_call(const char* what, const void* q, const void* k_pages, const void* v_pages, int64_t num_pages,
                  int kv_heads, const void* block_table, int bt_stride, const void* seq_lens, int B, int T,
                  const void* selected_idx, int k, float scale, float k_scale, float v_scale, const void* out,
                  const void* ws, size_t ws_bytes, StepLayout* lay) {
  const bool sparse = selected_idx != nullptr;
  if (int rc = check_step_shape(B, T, bt_stride, k, sparse)) return rc;
  if (kv_heads < 1 || kv_heads > kMaxHeads)
    return set_error(MONO_ENOTSUP, "%s: kv_heads must be in [1, %d] (got %d)", what, kMaxHeads, kv_heads);
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out || !ws)
    return set_error(MONO_EINVAL, "%s: NULL buffer", what);
  if (num_pages < 1) return set_error(MONO_EINVAL, "%s: num_pages must be >= 1", what);
  if (!finite(scale)) return set_error(MONO_EINVAL, "%s: scale must be finite", what);
  if (bad_tensor_scale(k_scale) || bad_tensor_scale(v_scale))
    return set_error(MONO_EINVAL, "%s: k_scale and v_scale must be finite and > 0", what);
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16) || !aligned(ws, 256) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(selected_idx, 4))
    return set_error(MONO_EINVAL, "%s: q/pages/out need 16-byte, ws 256-byte, tables 4-byte alignment", what);
  *lay = step_layout(kModeAttn, B, T, kv_heads, bt_stride, sparse ? k : 0, sparse);
  if (ws_bytes < lay->total) return set_error(MONO_ENOSPC, "%s: workspace %zu B < %zu B", what, ws_bytes, lay->total);
  return MONO_OK;
}

int check_sparse_call(const char* what, const void* index_q, const void* index_pages, const void* q,
                      const void* k_pages, const void* v_pages, int64_t num_pages, int kv_heads,
                      const void* block_table, int bt_stride, const void* seq_lens, int B, int T, int k,
                      float scale, float k_scale, float v_scale, const void* selected_idx, const void* out,
                      const void* ws, size_t ws_bytes, StepLayout* lay) {
  if (int rc = check_step_shape(B, T, bt_stride, k, true)) return rc;
  if (kv_heads < 1 || kv_heads > kMaxHeads)
    return set_error(MONO_ENOTSUP, "%s: kv_heads must be in [1, %d] (got %d)", what, kMaxHeads, kv_heads);
  if (!index_q || !index_pages || !q || !k_pages || !v_pages || !block_table || !seq_lens || !selected_idx || !out ||
      !ws)
    return set_error(MONO_EINVAL, "%s: NULL buffer", what);
  if (num_pages < 1) return set_error(MONO_EINVAL, "%s: num_pages must be >= 1", what);
  if (!finite(scale)) return set_error(MONO_EINVAL, "%s: scale must be finite", what);
  if (bad_tensor_scale(k_scale) || bad_tensor_scale(v_scale))
    return set_error(MONO_EINVAL, "%s: k_scale and v_scale must be finite and > 0", what);
  if (!aligned(index_q, 16) || !aligned(index_pages, 16) || !aligned(q, 16) || !aligned(k_pages, 16) ||
      !aligned(v_pages, 16) || !aligned(out, 16) || !aligned(ws, 256) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(selected_idx, 4))
    return set_error(MONO_EINVAL, "%s: q/pages/out need 16-byte, ws 256-byte, tables 4-byte alignment", what);
  *lay = step_layout(kModeFused, B, T, kv_heads, bt_stride, k, 1);
  if (ws_bytes < lay->total) return set_error(MONO_ENOSPC, "%s: workspace %zu B < %zu B", what, ws_bytes, lay->total);
  return MONO_OK;
}

int check_merge_call(const void* cand_idx, const void* cand_scores, int G, int64_t N, int k_in, int k_out,
                     const void* out_idx, const void* out_scores) {
  if (G < 1 || k_in < 1 || k_out < 1 || N < 0 || N > 0x7fffffff)
    return set_error(MONO_EINVAL, "mono_topk_merge: need G, k_in, k_out >= 1 and 0 <= N < 2^31");
  if ((int64_t)G * k_in > kMergeMaxCandidates)
    return set_error(MONO_ENOTSUP, "mono_topk_merge: G * k_in = %lld exceeds %d candidates", (long long)G * k_in,
                     kMergeMaxCandidates);
  if (N == 0) return MONO_OK;
  if (!cand_idx || !cand_scores || !out_idx) return set_error(MONO_EINVAL, "mono_topk_merge: NULL buffer");
  if (!aligned(cand_idx, 4) || !aligned(cand_scores, 4) || !aligned(out_idx, 4) || !aligned(out_scores, 4))
    return set_error(MONO_EINVAL, "mono_topk_merge: buffers need 4-byte alignment");
  return MONO_OK;
}

CpLayout cp_layout(int B, int T, int G, int bt_stride, int k, int shards) {
  CpLayout c{};
  c.index = step_layout(kModeIndex, B, T, 1, bt_stride, k, 1, G);
  c.width = (bt_stride + shards - 1) / shards;
  c.shards = (bt_stride + c.width - 1) / c.width;  // windows [r * width, ...) that start inside the table
  const size_t rows = (size_t)G * B * T;
  const size_t cand = (size_t)c.shards * rows * (size_t)k * 4;
  c.cand_idx = (c.index.total + 255) & ~(size_t)255;
  c.cand_scores = c.cand_idx + ((cand + 255) & ~(size_t)255);
  c.total = c.cand_scores + cand;
  return c;
}

int check_cp_call(const void* index_q, const void* index_pages, int64_t num_pages, const void* block_table,
                  int bt_stride, const void* seq_lens, int B, int T, int G, int k, int shards, const void* out,
                  const void* ws, size_t ws_bytes, CpLayout* lay) {
  const char* what = "mono_indexer_cp_topk";
  if (int rc = check_step_shape(B, T, bt_stride, k, true)) return rc;
  if (G < 1 || G > kMaxHeads) return set_error(MONO_EINVAL, "%s: heads must be in [1, %d] (got %d)", what, kMaxHeads, G);
  if ((long long)G * B * T > (1LL << 30)) return set_error(MONO_EINVAL, "%s: heads*B*T too large", what);
  if (shards < 1 || shards > 65536) return set_error(MONO_EINVAL, "%s: shards must be in [1, 65536] (got %d)", what, shards);
  if (!index_q || !index_pages || !block_table || !seq_lens || !out || !ws)
    return set_error(MONO_EINVAL, "%s: NULL buffer", what);
  if (num_pages < 1) return set_error(MONO_EINVAL, "%s: num_pages must be >= 1", what);
  if (!aligned(index_q, 16) || !aligned(index_pages, 16) || !aligned(ws, 256) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(out, 4))
    return set_error(MONO_EINVAL, "%s: index_q/pages need 16-byte, ws 256-byte, tables 4-byte alignment", what);
  *lay = cp_layout(B, T, G, bt_stride, k, shards);
  if ((long long)lay->shards * k > kMergeMaxCandidates)
    return set_error(MONO_ENOTSUP, "%s: shards*k = %d*%d candidates per row exceed %d", what, lay->shards, k,
                     kMergeMaxCandidates);
  if (ws_bytes < lay->total) return set_error(MONO_ENOSPC, "%s: workspace %zu B < %zu B", what, ws_bytes, lay->total);
  return MONO_OK;
}

int check_insert_call(const void* k_rows, const void* v_rows, const void* index_rows, const void* slots, int64_t n,
                      int kv_heads, const void* k_pages, const void* v_pages, const void* index_pages,
                      int64_t num_pages, const void* err) {
  if (n < 0) return set_error(MONO_EINVAL, "mono_insert_mxfp4: n < 0");
  if (num_pages < 1 || num_pages > ((int64_t)1 << 34))
    return set_error(MONO_EINVAL, "mono_insert_mxfp4: num_pages out of range");
  if ((k_rows == nullptr) != (k_pages == nullptr) || (v_rows == nullptr) != (v_pages == nullptr) ||
      (index_rows == nullptr) != (index_pages == nullptr))
    return set_error(MONO_EINVAL, "mono_insert_mxfp4: rows and pages of a cache must be both given or both NULL");
  const bool kv = k_rows || v_rows;
  if (kv && (kv_heads < 1 || kv_heads > kMaxHeads))
    return set_error(MONO_ENOTSUP, "mono_insert_mxfp4: kv_heads must be in [1, %d] (got %d)", kMaxHeads, kv_heads);
  if (!slots || !err) return set_error(MONO_EINVAL, "mono_insert_mxfp4: NULL slots or err");
  const void* bufs16[6] = {k_rows, v_rows, index_rows, k_pages, v_pages, index_pages};
  for (const void* b : bufs16)
    if (b && !aligned(b, 16)) return set_error(MONO_EINVAL, "mono_insert_mxfp4: rows and pages need 16-byte alignment");
  if (!aligned(slots, 8) || !aligned(err, 4))
    return set_error(MONO_EINVAL, "mono_insert_mxfp4: slots need 8-byte and err 4-byte alignment");
  // n x rows per token x 4 must stay below 2^31 (checked without forming the product)
  const int64_t rows_per_token = (k_rows ? kv_heads : 0) + (v_rows ? kv_heads : 0) + (index_rows ? 1 : 0);
  if (rows_per_token > 0 && n >= (((int64_t)1 << 31) + rows_per_token * 4 - 1) / (rows_per_token * 4))
    return set_error(MONO_EINVAL, "mono_insert_mxfp4: n x rows per token too large");
  return MONO_OK;
}

int check_bench_read_call(const void* pages, const void* page_ids, int64_t n_pages, int mode, int grid,
                          const void* sink) {
  if (mode != 0 && mode != 1) return set_error(MONO_EINVAL, "mono_bench_read: mode must be 0 or 1 (got %d)", mode);
  if (n_pages < 1 || n_pages > ((int64_t)1 << 30))
    return set_error(MONO_EINVAL, "mono_bench_read: n_pages out of range");
  if (grid < 1 || grid > (1 << 16)) return set_error(MONO_EINVAL, "mono_bench_read: grid must be in [1, 65536]");
  if (!pages || !sink || (mode == 1 && !page_ids)) return set_error(MONO_EINVAL, "mono_bench_read: NULL buffer");
  if (!aligned(pages, 16) || !aligned(sink, 4) || !aligned(page_ids, 4))
    return set_error(MONO_EINVAL, "mono_bench_read: pages need 16-byte, ids and sink 4-byte alignment");
  return MONO_OK;
}

int check_bench_scan_call(const void* index_q, const void* pages, int64_t num_pages, const void* block_table,
                          int bt_stride, const void* seq_lens, int B, int chunk_pages, int variant, const void* hist,
                          const void* err) {
  const char* what = "mono_bench_scan";
  if (variant != 0 && variant != 1) return set_error(MONO_EINVAL, "%s: variant must be 0 or 1 (got %d)", what, variant);
  if (B < 1 || B > (1 << 16)) return set_error(MONO_EINVAL, "%s: B must be in [1, 65536]", what);
  if (bt_stride < 1 || bt_stride > kMaxBtStride) return set_error(MONO_EINVAL, "%s: bad bt_stride %d", what, bt_stride);
  if (chunk_pages < 1 || chunk_pages * kPageTokens > kLocalTokens)
    return set_error(MONO_EINVAL, "%s: chunk_pages must be in [1, %d]", what, kLocalTokens / kPageTokens);
  if ((int64_t)B * ((bt_stride + chunk_pages - 1) / chunk_pages) > ((int64_t)1 << 30))
    return set_error(MONO_EINVAL, "%s: too many workgroups", what);
  if (num_pages < 1) return set_error(MONO_EINVAL, "%s: num_pages must be >= 1", what);
  if (!index_q || !pages || !block_table || !seq_lens || !hist || !err)
    return set_error(MONO_EINVAL, "%s: NULL buffer", what);
  if (!aligned(index_q, 16) || !aligned(pages, 16) || !aligned(block_table, 4) || !aligned(seq_lens, 4) ||
      !aligned(hist, 4) || !aligned(err, 4))
    return set_error(MONO_EINVAL, "%s: index_q/pages need 16-byte, tables and outputs 4-byte alignment", what);
  return MONO_OK;
}

}  // namespace mono
