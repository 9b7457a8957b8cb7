// C ABI of libmono_decode.so: argument validation, error reporting and the
// calls into the kernel launchers.  The contract of every entry point is in
// include/mono_decode.h.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <vector>

#include "mono_decode.h"
#include "launch.h"

#include <algorithm>

namespace mono {

namespace {
// Optional per-kernel timing: pairs of HIP events recorded around launches.
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> ev;  // 2 per slot
  std::vector<int> kid;        // kernel id per slot
  int used = 0;
};
Profiler g_prof;
// The step kernel is one kernel; it is timed under the name of the call.
const char* const kKernelNames[kNumKernels] = {
    "pack_kernel",          "unpack_kernel",         "dequant_f32_kernel",  "dequant_bf16_kernel",
    "index_topk_kernel",    "pa_decode_kernel",      "sparse_decode_kernel", "insert_kernel",
    "index_topk_fp8_kernel", "pa_decode_fp8_kernel", "sparse_decode_fp8_kernel", "dequant_fp8_bf16_kernel",
    "topk_merge_kernel",    "read_stream_kernel",    "read_gather_kernel", "scan_mfma_kernel",
    "scan_valu_kernel"};
}  // namespace

bool prof_slot(int id, hipEvent_t* start, hipEvent_t* stop) {
  if (!g_prof.on) return false;
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (!g_prof.on || g_prof.used >= (int)g_prof.kid.size()) return false;
  const int sl = g_prof.used++;
  g_prof.kid[sl] = id;
  *start = g_prof.ev[2 * sl];
  *stop = g_prof.ev[2 * sl + 1];
  return true;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MONO_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return MONO_OK;
}

namespace {

int index_topk_impl(int fmt, const char* what, const uint16_t* index_q_dev, const uint8_t* index_pages_dev,
                    int64_t num_pages, const int32_t* block_table_dev, int bt_stride, const int32_t* seq_lens_dev,
                    int B, int T, int k, int32_t* selected_idx_dev, float* selected_scores_dev, void* ws_dev,
                    size_t ws_bytes, void* stream, int page_lo = 0, int page_hi = -1) {
  clear_error();
  StepLayout lay;
  if (int rc = check_index_call(what, index_q_dev, index_pages_dev, num_pages, block_table_dev, bt_stride,
                                seq_lens_dev, B, T, k, selected_idx_dev, selected_scores_dev, ws_dev, ws_bytes,
                                page_lo, page_hi, &lay))
    return rc;
  StepArgs a{};
  a.fmt = fmt;
  a.index_q = index_q_dev;
  a.index_pages = index_pages_dev;
  a.num_pages = num_pages;
  a.block_table = block_table_dev;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens_dev;
  a.sel = selected_idx_dev;
  a.sel_scores = selected_scores_dev;
  a.ws = static_cast<uint8_t*>(ws_dev);
  return launch_step(a, lay, (hipStream_t)stream, what);
}

int pa_decode_impl(int fmt, const char* what, const uint16_t* q_dev, const uint8_t* k_pages_dev,
                   const uint8_t* v_pages_dev, int64_t num_pages, int kv_heads, const int32_t* block_table_dev,
                   int bt_stride, const int32_t* seq_lens_dev, int B, int T, const int32_t* selected_idx_dev, int k,
                   float scale, float k_scale, float v_scale, uint16_t* out_dev, void* ws_dev, size_t ws_bytes,
                   void* stream) {
  clear_error();
  StepLayout lay;
  if (int rc = check_pa_call(what, q_dev, k_pages_dev, v_pages_dev, num_pages, kv_heads, block_table_dev, bt_stride,
                             seq_lens_dev, B, T, selected_idx_dev, k, scale, k_scale, v_scale, out_dev, ws_dev,
                             ws_bytes, &lay))
    return rc;
  StepArgs a{};
  a.fmt = fmt;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.q = q_dev;
  a.k_pages = k_pages_dev;
  a.v_pages = v_pages_dev;
  a.num_pages = num_pages;
  a.block_table = block_table_dev;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens_dev;
  a.sel = const_cast<int32_t*>(selected_idx_dev);
  a.scale = scale;
  a.out = out_dev;
  a.ws = static_cast<uint8_t*>(ws_dev);
  return launch_step(a, lay, (hipStream_t)stream, what);
}

int sparse_decode_impl(int fmt, const char* what, const uint16_t* index_q_dev, const uint8_t* index_pages_dev,
                       const uint16_t* q_dev, const uint8_t* k_pages_dev, const uint8_t* v_pages_dev,
                       int64_t num_pages, int kv_heads, const int32_t* block_table_dev, int bt_stride,
                       const int32_t* seq_lens_dev, int B, int T, int k, float scale, float k_scale, float v_scale,
                       int32_t* selected_idx_dev, uint16_t* out_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  clear_error();
  StepLayout lay;
  if (int rc = check_sparse_call(what, index_q_dev, index_pages_dev, q_dev, k_pages_dev, v_pages_dev, num_pages,
                                 kv_heads, block_table_dev, bt_stride, seq_lens_dev, B, T, k, scale, k_scale, v_scale,
                                 selected_idx_dev, out_dev, ws_dev, ws_bytes, &lay))
    return rc;
  StepArgs a{};
  a.fmt = fmt;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.index_q = index_q_dev;
  a.index_pages = index_pages_dev;
  a.q = q_dev;
  a.k_pages = k_pages_dev;
  a.v_pages = v_pages_dev;
  a.num_pages = num_pages;
  a.block_table = block_table_dev;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens_dev;
  a.sel = selected_idx_dev;
  a.scale = scale;
  a.out = out_dev;
  a.ws = static_cast<uint8_t*>(ws_dev);
  return launch_step(a, lay, (hipStream_t)stream, what);
}

}  // namespace
}  // namespace mono

using namespace mono;

extern "C" {

int mono_abi_version(void) { return MONO_ABI_VERSION; }

const char* mono_last_error(void) { return last_error(); }

int mxfp4_pages_pack(const uint8_t* codes_dev, const uint8_t* scales_dev, uint8_t* pages_dev,
                     int64_t n_pages, void* stream) {
  clear_error();
  if (int rc = check_pages_args(codes_dev, scales_dev, pages_dev, n_pages, 16, 4, 16, "mxfp4_pages_pack")) return rc;
  if (n_pages == 0) return MONO_OK;
  return launch_pack(codes_dev, scales_dev, pages_dev, n_pages, (hipStream_t)stream);
}

int mxfp4_pages_unpack(const uint8_t* pages_dev, uint8_t* codes_dev, uint8_t* scales_dev,
                       int64_t n_pages, void* stream) {
  clear_error();
  if (int rc = check_pages_args(pages_dev, codes_dev, scales_dev, n_pages, 16, 16, 4, "mxfp4_pages_unpack")) return rc;
  if (n_pages == 0) return MONO_OK;
  return launch_unpack(pages_dev, codes_dev, scales_dev, n_pages, (hipStream_t)stream);
}

int mxfp4_pages_dequant(const uint8_t* pages_dev, float* out_dev, int64_t n_pages, void* stream) {
  clear_error();
  if (int rc = check_pages_args(pages_dev, out_dev, out_dev, n_pages, 16, 16, 16, "mxfp4_pages_dequant")) return rc;
  if (n_pages == 0) return MONO_OK;
  return launch_dequant_f32(pages_dev, out_dev, n_pages, (hipStream_t)stream);
}

int mxfp4_pages_dequant_bf16(const uint8_t* pages_dev, uint16_t* out_dev, int64_t n_pages, void* stream) {
  clear_error();
  if (int rc = check_pages_args(pages_dev, out_dev, out_dev, n_pages, 16, 16, 16, "mxfp4_pages_dequant_bf16")) return rc;
  if (n_pages == 0) return MONO_OK;
  return launch_dequant_bf16(pages_dev, out_dev, n_pages, (hipStream_t)stream);
}

size_t mono_index_score_topk_workspace(int B, int T, int bt_stride, int k) {
  if (check_step_shape(B, T, bt_stride, k, true) != MONO_OK) return 0;
  return step_layout(kModeIndex, B, T, 1, bt_stride, k, 1).total;
}

int mono_index_score_topk(const uint16_t* index_q_dev, const uint8_t* index_pages_dev, int64_t num_pages,
                          const int32_t* block_table_dev, int bt_stride, const int32_t* seq_lens_dev,
                          int B, int T, int k, int32_t* selected_idx_dev, float* selected_scores_dev,
                          void* ws_dev, size_t ws_bytes, void* stream) {
  return index_topk_impl(kFmtMxfp4, "mono_index_score_topk", index_q_dev, index_pages_dev, num_pages, block_table_dev,
                         bt_stride, seq_lens_dev, B, T, k, selected_idx_dev, selected_scores_dev, ws_dev, ws_bytes,
                         stream);
}

int mono_index_score_topk_window(const uint16_t* index_q_dev, const uint8_t* index_pages_dev, int64_t num_pages,
                                 const int32_t* block_table_dev, int bt_stride, const int32_t* seq_lens_dev, int B,
                                 int T, int k, int page_lo, int page_hi, int32_t* selected_idx_dev,
                                 float* selected_scores_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  return index_topk_impl(kFmtMxfp4, "mono_index_score_topk_window", index_q_dev, index_pages_dev, num_pages,
                         block_table_dev, bt_stride, seq_lens_dev, B, T, k, selected_idx_dev, selected_scores_dev,
                         ws_dev, ws_bytes, stream, page_lo, page_hi);
}

int mono_topk_merge(const int32_t* cand_idx_dev, const float* cand_scores_dev, int G, int64_t N, int k_in, int k_out,
                    int32_t* out_idx_dev, float* out_scores_dev, void* stream) {
  clear_error();
  if (int rc = check_merge_call(cand_idx_dev, cand_scores_dev, G, N, k_in, k_out, out_idx_dev, out_scores_dev))
    return rc;
  if (N == 0) return MONO_OK;
  return launch_topk_merge(cand_idx_dev, cand_scores_dev, G, (int)N, k_in, k_out, out_idx_dev, out_scores_dev,
                           (hipStream_t)stream);
}

size_t mono_indexer_cp_topk_workspace(int B, int T, int heads, int bt_stride, int k, int shards) {
  if (check_step_shape(B, T, bt_stride, k, true) != MONO_OK || heads < 1 || heads > kMaxHeads || shards < 1 ||
      shards > 65536)
    return 0;
  return cp_layout(B, T, heads, bt_stride, k, shards).total;
}

int mono_indexer_cp_topk(const uint16_t* index_q_dev, const uint8_t* index_pages_dev, int64_t num_pages,
                         const int32_t* block_table_dev, int bt_stride, const int32_t* seq_lens_dev, int B, int T,
                         int heads, int k, int shards, int32_t* selected_idx_dev, void* ws_dev, size_t ws_bytes,
                         void* stream) {
  const char* what = "mono_indexer_cp_topk";
  clear_error();
  CpLayout cp;
  if (int rc = check_cp_call(index_q_dev, index_pages_dev, num_pages, block_table_dev, bt_stride, seq_lens_dev, B, T,
                             heads, k, shards, selected_idx_dev, ws_dev, ws_bytes, &cp))
    return rc;
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  int32_t* cand = reinterpret_cast<int32_t*>(ws + cp.cand_idx);
  float* cand_s = reinterpret_cast<float*>(ws + cp.cand_scores);
  const size_t rows = (size_t)heads * B * T;
  StepArgs a{};
  a.fmt = kFmtMxfp4;
  a.index_q = index_q_dev;
  a.index_pages = index_pages_dev;
  a.num_pages = num_pages;
  a.block_table = block_table_dev;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens_dev;
  a.ws = ws;
  // Shard r scores its page window for every head in one launch (each
  // window page is read once), into its own candidate lists.
  for (int r = 0; r < cp.shards; ++r) {
    StepLayout lay = cp.index;
    lay.win_lo = r * cp.width;
    lay.win_hi = std::min(bt_stride, (r + 1) * cp.width);
    a.sel = cand + (size_t)r * rows * k;
    a.sel_scores = cand_s + (size_t)r * rows * k;
    if (int rc = launch_step(a, lay, (hipStream_t)stream, what)) return rc;
  }
  // Each head's owner keeps the top k of the shards' lists.
  return launch_topk_merge(cand, cand_s, cp.shards, (int)rows, k, k, selected_idx_dev, nullptr, (hipStream_t)stream);
}

int mono_index_score_topk_fp8(const uint16_t* index_q_dev, const uint8_t* index_pages_dev, int64_t num_pages,
                              const int32_t* block_table_dev, int bt_stride, const int32_t* seq_lens_dev, int B,
                              int T, int k, int32_t* selected_idx_dev, float* selected_scores_dev, void* ws_dev,
                              size_t ws_bytes, void* stream) {
  return index_topk_impl(kFmtFp8, "mono_index_score_topk_fp8", index_q_dev, index_pages_dev, num_pages,
                         block_table_dev, bt_stride, seq_lens_dev, B, T, k, selected_idx_dev, selected_scores_dev,
                         ws_dev, ws_bytes, stream);
}

size_t mono_pa_decode_workspace(int B, int T, int kv_heads, int bt_stride, int k, int sparse) {
  if (check_step_shape(B, T, bt_stride, k, sparse != 0) != MONO_OK) return 0;
  if (kv_heads < 1 || kv_heads > kMaxHeads) return 0;
  return step_layout(kModeAttn, B, T, kv_heads, bt_stride, sparse ? k : 0, sparse != 0).total;
}

int mono_pa_decode_mxfp4(const uint16_t* q_dev, const uint8_t* k_pages_dev, const uint8_t* v_pages_dev,
                         int64_t num_pages, int kv_heads, const int32_t* block_table_dev, int bt_stride,
                         const int32_t* seq_lens_dev, int B, int T, const int32_t* selected_idx_dev, int k,
                         float scale, uint16_t* out_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  return pa_decode_impl(kFmtMxfp4, "mono_pa_decode_mxfp4", q_dev, k_pages_dev, v_pages_dev, num_pages, kv_heads,
                        block_table_dev, bt_stride, seq_lens_dev, B, T, selected_idx_dev, k, scale, 1.f, 1.f, out_dev,
                        ws_dev, ws_bytes, stream);
}

int mono_pa_decode_fp8(const uint16_t* q_dev, const uint8_t* k_pages_dev, const uint8_t* v_pages_dev,
                       int64_t num_pages, int kv_heads, const int32_t* block_table_dev, int bt_stride,
                       const int32_t* seq_lens_dev, int B, int T, const int32_t* selected_idx_dev, int k, float scale,
                       float k_scale, float v_scale, uint16_t* out_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  return pa_decode_impl(kFmtFp8, "mono_pa_decode_fp8", q_dev, k_pages_dev, v_pages_dev, num_pages, kv_heads,
                        block_table_dev, bt_stride, seq_lens_dev, B, T, selected_idx_dev, k, scale, k_scale, v_scale,
                        out_dev, ws_dev, ws_bytes, stream);
}

size_t mono_sparse_decode_workspace(int B, int T, int kv_heads, int bt_stride, int k) {
  if (check_step_shape(B, T, bt_stride, k, true) != MONO_OK) return 0;
  if (kv_heads < 1 || kv_heads > kMaxHeads) return 0;
  return step_layout(kModeFused, B, T, kv_heads, bt_stride, k, 1).total;
}

int mono_sparse_decode_mxfp4(const uint16_t* index_q_dev, const uint8_t* index_pages_dev, const uint16_t* q_dev,
                             const uint8_t* k_pages_dev, const uint8_t* v_pages_dev, int64_t num_pages,
                             int kv_heads, const int32_t* block_table_dev, int bt_stride,
                             const int32_t* seq_lens_dev, int B, int T, int k, float scale,
                             int32_t* selected_idx_dev, uint16_t* out_dev, void* ws_dev, size_t ws_bytes,
                             void* stream) {
  return sparse_decode_impl(kFmtMxfp4, "mono_sparse_decode_mxfp4", index_q_dev, index_pages_dev, q_dev, k_pages_dev,
                            v_pages_dev, num_pages, kv_heads, block_table_dev, bt_stride, seq_lens_dev, B, T, k, scale,
                            1.f, 1.f, selected_idx_dev, out_dev, ws_dev, ws_bytes, stream);
}

int mono_sparse_decode_mxfp4_noalloc(const uint16_t* index_q_dev, const uint8_t* index_pages_dev,
                                     const uint16_t* q_dev, const uint8_t* k_pages_dev,
                                     const uint8_t* v_pages_dev, int64_t num_pages, int kv_heads,
                                     const int32_t* block_table_dev, int bt_stride, const int32_t* seq_lens_dev,
                                     int B, int T, int k, float scale, int32_t* selected_idx_dev,
                                     uint16_t* out_dev, uint32_t* err_dev, void* stream) {
  clear_error();
  const char* what = "mono_sparse_decode_mxfp4_noalloc";
  if (int rc = check_step_shape(B, T, bt_stride, k, true)) return rc;
  if (kv_heads < 1 || kv_heads > kMaxHeads)
    return set_error(MONO_ENOTSUP, "%s: kv_heads must be in [1, %d] (got %d)", what, kMaxHeads, kv_heads);
  if ((uintptr_t)err_dev % 4) return set_error(MONO_EINVAL, "%s: err needs 4-byte alignment", what);
  const StepLayout lay = step_layout(kModeFused, B, T, kv_heads, bt_stride, k, 1);
  if (lay.total > kNoAllocScratchBytes)
    return set_error(MONO_ENOSPC, "%s: this shape needs %zu B of scratch; the static scratch holds %zu B", what,
                     lay.total, kNoAllocScratchBytes);
  uint8_t* ws = nullptr;
  if (int rc = noalloc_scratch((hipStream_t)stream, &ws)) return rc;
  if (int rc = sparse_decode_impl(kFmtMxfp4, what, index_q_dev, index_pages_dev, q_dev, k_pages_dev, v_pages_dev,
                                  num_pages, kv_heads, block_table_dev, bt_stride, seq_lens_dev, B, T, k, scale, 1.f,
                                  1.f, selected_idx_dev, out_dev, ws, kNoAllocScratchBytes, stream))
    return rc;
  return err_dev ? launch_scratch_errors(ws, lay.err, err_dev, (hipStream_t)stream) : MONO_OK;
}

int mono_sparse_decode_fp8(const uint16_t* index_q_dev, const uint8_t* index_pages_dev, const uint16_t* q_dev,
                           const uint8_t* k_pages_dev, const uint8_t* v_pages_dev, int64_t num_pages, int kv_heads,
                           const int32_t* block_table_dev, int bt_stride, const int32_t* seq_lens_dev, int B, int T,
                           int k, float scale, float k_scale, float v_scale, int32_t* selected_idx_dev,
                           uint16_t* out_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  return sparse_decode_impl(kFmtFp8, "mono_sparse_decode_fp8", index_q_dev, index_pages_dev, q_dev, k_pages_dev,
                            v_pages_dev, num_pages, kv_heads, block_table_dev, bt_stride, seq_lens_dev, B, T, k, scale,
                            k_scale, v_scale, selected_idx_dev, out_dev, ws_dev, ws_bytes, stream);
}

int fp8_pages_dequant_bf16(const uint8_t* pages_dev, uint16_t* out_dev, int64_t n_pages, void* stream) {
  clear_error();
  if (int rc = check_pages_args(pages_dev, out_dev, out_dev, n_pages, 16, 16, 16, "fp8_pages_dequant_bf16")) return rc;
  if (n_pages == 0) return MONO_OK;
  return launch_dequant_fp8_bf16(pages_dev, out_dev, n_pages, (hipStream_t)stream);
}

int mono_insert_mxfp4(const uint16_t* k_rows_dev, const uint16_t* v_rows_dev, const uint16_t* index_rows_dev,
                      const int64_t* slots_dev, int64_t n, int kv_heads, uint8_t* k_pages_dev, uint8_t* v_pages_dev,
                      uint8_t* index_pages_dev, int64_t num_pages, uint32_t* err_dev, void* stream) {
  clear_error();
  if (int rc = check_insert_call(k_rows_dev, v_rows_dev, index_rows_dev, slots_dev, n, kv_heads, k_pages_dev,
                                 v_pages_dev, index_pages_dev, num_pages, err_dev))
    return rc;
  const int row_heads[3] = {k_rows_dev ? kv_heads : 0, v_rows_dev ? kv_heads : 0, index_rows_dev ? 1 : 0};
  const int64_t rows_per_token = row_heads[0] + row_heads[1] + row_heads[2];
  if (n == 0 || rows_per_token == 0) return MONO_OK;
  const uint16_t* const rows[3] = {k_rows_dev, v_rows_dev, index_rows_dev};
  uint8_t* const pools[3] = {k_pages_dev, v_pages_dev, index_pages_dev};
  return launch_insert(rows, pools, row_heads, slots_dev, n, num_pages, err_dev, (hipStream_t)stream);
}

int mono_bench_read(const uint8_t* pages_dev, const int32_t* page_ids_dev, int64_t n_pages, int mode, int grid,
                    uint32_t* sink_dev, void* stream) {
  clear_error();
  if (int rc = check_bench_read_call(pages_dev, page_ids_dev, n_pages, mode, grid, sink_dev)) return rc;
  return launch_read_reference(pages_dev, page_ids_dev, n_pages, mode, grid, sink_dev, (hipStream_t)stream);
}

int mono_profile_start(int capacity) {
  clear_error();
  if (capacity < 1 || capacity > (1 << 20)) return set_error(MONO_EINVAL, "mono_profile_start: capacity out of range");
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (g_prof.on) return set_error(MONO_EINVAL, "mono_profile_start: already started");
  g_prof.ev.assign(2 * (size_t)capacity, nullptr);
  g_prof.kid.assign((size_t)capacity, -1);
  for (auto& e : g_prof.ev) {
    if (hipEventCreate(&e) != hipSuccess) return set_error(MONO_EHIP, "mono_profile_start: hipEventCreate failed");
  }
  g_prof.used = 0;
  g_prof.on = true;
  return MONO_OK;
}

int mono_profile_stop(double* total_ms, int* launches, int n_kernels) {
  clear_error();
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (!g_prof.on) return set_error(MONO_EINVAL, "mono_profile_stop: not started");
  g_prof.on = false;
  int rc = MONO_OK;
  for (int k = 0; k < n_kernels && total_ms && launches; ++k) {
    total_ms[k] = 0.0;
    launches[k] = 0;
  }
  for (int sl = 0; sl < g_prof.used; ++sl) {
    float ms = 0.f;
    if (hipEventSynchronize(g_prof.ev[2 * sl + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof.ev[2 * sl], g_prof.ev[2 * sl + 1]) != hipSuccess) {
      rc = set_error(MONO_EHIP, "mono_profile_stop: event timing failed");
      break;
    }
    const int k = g_prof.kid[sl];
    if (k >= 0 && k < n_kernels && total_ms && launches) {
      total_ms[k] += ms;
      launches[k] += 1;
    }
  }
  for (auto& e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.kid.clear();
  g_prof.used = 0;
  return rc == MONO_OK ? kNumKernels : rc;
}

int mono_bench_scan(const uint16_t* index_q_dev, const uint8_t* index_pages_dev, int64_t num_pages,
                    const int32_t* block_table_dev, int bt_stride, const int32_t* seq_lens_dev, int B, int chunk_pages,
                    int variant, uint32_t* hist_dev, uint32_t* err_dev, void* stream) {
  clear_error();
  if (int rc = check_bench_scan_call(index_q_dev, index_pages_dev, num_pages, block_table_dev, bt_stride,
                                     seq_lens_dev, B, chunk_pages, variant, hist_dev, err_dev))
    return rc;
  return launch_bench_scan(index_q_dev, index_pages_dev, num_pages, block_table_dev, bt_stride, seq_lens_dev, B,
                           chunk_pages, variant, hist_dev, err_dev, (hipStream_t)stream);
}

const char* mono_kernel_name(int id) { return (id >= 0 && id < kNumKernels) ? kKernelNames[id] : ""; }

int mono_check_device_errors(void* ws_dev, void* stream) {
  clear_error();
  if (!ws_dev) return set_error(MONO_EINVAL, "mono_check_device_errors: NULL workspace");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  uint32_t bits = 0;
  if (e == hipSuccess) e = hipMemcpy(&bits, ws_dev, sizeof(bits), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(ws_dev, 0, sizeof(bits));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return set_error(MONO_EHIP, "mono_check_device_errors: %s", hipGetErrorString(e));
  return (int)(bits & 0x7fffffffu);
}

}  // extern "C"
