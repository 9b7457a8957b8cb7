// Host-side launch interface between the C ABI layer (abi.hip) and the
// kernel files.  Every launcher only enqueues work on `stream`.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mono {

// Records `what` and the pending HIP launch error (if any) as the thread's
// last error; returns MONO_OK or MONO_EHIP.
int check_launch(const char* what);

// Kernel ids of the optional per-kernel event timing (mono_profile_*).
enum KernelId { kKPack = 0, kKUnpack, kKDequant, kKDequantBf16, kKIndexScan, kKTopkFilter, kKPaDecode, kNumKernels };
// When timing is on, takes the next pair of timing events for kernel `id`
// and returns true; the launch then records them as part of its dispatch.
bool prof_slot(int id, hipEvent_t* start, hipEvent_t* stop);

// Launch through hipExtLaunchKernelGGL with dispatch-attached start/stop
// events while per-kernel timing is on, plain hipLaunchKernelGGL otherwise.
#define MONO_LAUNCH(ID, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                              \
  do {                                                                                       \
    hipEvent_t mono_ev0_ = nullptr, mono_ev1_ = nullptr;                                     \
    if (::mono::prof_slot((ID), &mono_ev0_, &mono_ev1_))                                     \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, mono_ev0_, mono_ev1_, 0u,    \
                            __VA_ARGS__);                                                    \
    else                                                                                     \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                   \
  } while (0)
// Records a formatted error message; returns `code`.
int set_error(int code, const char* fmt, ...);

int launch_pack(const uint8_t* codes, const uint8_t* scales, uint8_t* pages, int64_t n_pages,
                hipStream_t stream);
int launch_unpack(const uint8_t* pages, uint8_t* codes, uint8_t* scales, int64_t n_pages,
                  hipStream_t stream);
int launch_dequant_f32(const uint8_t* pages, float* out, int64_t n_pages, hipStream_t stream);
int launch_dequant_bf16(const uint8_t* pages, uint16_t* out, int64_t n_pages, hipStream_t stream);

// ---- index scoring + top-k ----------------------------------------------------
struct TopkLayout {
  size_t err, flt_cnt, out_cnt, cand_cnt, hist, scores, cand, total;
  int q_groups;  // ceil(T / 4)
  int lcap;      // bt_stride * 128
};
TopkLayout topk_layout(int B, int T, int bt_stride, int k);

struct TopkArgs {
  const uint16_t* index_q;
  const uint8_t* pages;
  int64_t num_pages;
  const int32_t* block_table;
  int bt_stride;
  const int32_t* seq_lens;
  int B, T, k;
  int32_t* selected_idx;
  float* selected_scores;
  uint8_t* ws;
};
int launch_index_topk(const TopkArgs& a, const TopkLayout& lay, hipStream_t stream);

// ---- paged decode attention ---------------------------------------------------
struct PaLayout {
  size_t err, cnt, pm, pl, pacc, total;
  int split_tokens;  // list entries per workgroup
  int n_splits;      // workgroups per (query token, KV head)
};
PaLayout pa_layout(int B, int T, int kv_heads, int bt_stride, int k, int sparse);

struct PaArgs {
  const uint16_t* q;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  int64_t num_pages;
  int kv_heads;
  const int32_t* block_table;
  int bt_stride;
  const int32_t* seq_lens;
  int B, T;
  const int32_t* selected_idx;
  int k;
  float scale;
  uint16_t* out;
  uint8_t* ws;
};
int launch_pa_decode(const PaArgs& a, const PaLayout& lay, hipStream_t stream);

}  // namespace mono
