// Host-side launch interface between the C ABI layer (abi.hip) and the
// kernel files.  Every launcher only enqueues work on `stream`.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mono_decode.h"
#include "plan.h"

namespace mono {

// Records `what` and the pending HIP launch error (if any) as the thread's
// last error; returns MONO_OK or MONO_EHIP.
int check_launch(const char* what);

// Kernel ids of the optional per-kernel event timing (mono_profile_*).
enum KernelId {
  kKPack = 0,
  kKUnpack,
  kKDequant,
  kKDequantBf16,
  kKIndexScan,
  kKPaDecode,
  kKStep,
  kKInsert,
  kKIndexScanFp8,
  kKPaDecodeFp8,
  kKStepFp8,
  kKDequantFp8Bf16,
  kKTopkMerge,
  kKReadStream,
  kKReadGather,
  kKScanMfma,
  kKScanValu,
  kNumKernels
};
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

int launch_pack(const uint8_t* codes, const uint8_t* scales, uint8_t* pages, int64_t n_pages,
                hipStream_t stream);
int launch_unpack(const uint8_t* pages, uint8_t* codes, uint8_t* scales, int64_t n_pages,
                  hipStream_t stream);
int launch_dequant_f32(const uint8_t* pages, float* out, int64_t n_pages, hipStream_t stream);
int launch_dequant_bf16(const uint8_t* pages, uint16_t* out, int64_t n_pages, hipStream_t stream);
// Merge of G per-shard top-k lists per query token (merge.hip): candidates
// [G, N, k_in] (positions, -1 = empty; fp32 scores) -> [N, k_out].
int launch_topk_merge(const int32_t* cand_idx, const float* cand_scores, int G, int N, int k_in, int k_out,
                      int32_t* out_idx, float* out_scores, hipStream_t stream);
// Read-bandwidth references (bench_read.hip): mode 0 streams the bytes of
// n_pages pages, mode 1 gathers the pages page_ids[0..n_pages) with the
// index scan's lane pattern; grid workgroups, one word each to sink.
int launch_read_reference(const uint8_t* pages, const int32_t* page_ids, int64_t n_pages, int mode, int grid,
                          uint32_t* sink, hipStream_t stream);
// The index scan phase on the matrix cores (variant 0) or the VALU
// (variant 1), for benchmarks (bench_scan.hip).
int launch_bench_scan(const uint16_t* index_q, const uint8_t* pages, int64_t num_pages, const int32_t* block_table,
                      int bt_stride, const int32_t* seq_lens, int B, int chunk_pages, int variant, uint32_t* hist,
                      uint32_t* err, hipStream_t stream);
// fp8 pages [n_pages, 16384] -> bf16 [n_pages, 128, 128] through the step kernel's conversion.
int launch_dequant_fp8_bf16(const uint8_t* pages, uint16_t* out, int64_t n_pages, hipStream_t stream);
// Cache insert: caches c = 0 (K), 1 (V), 2 (index key) with row_heads[c]
// rows per token (0 = not written); rows[c] bf16 [n, row_heads[c], 128],
// pools[c] [num_pages, row_heads[c], 8704].
int launch_insert(const uint16_t* const rows[3], uint8_t* const pools[3], const int row_heads[3],
                  const int64_t* slots, int64_t n, int64_t num_pages, uint32_t* err, hipStream_t stream);

// ---- the persistent step kernel (step.hip); its layout is in plan.h -----------
struct StepArgs {
  int fmt = kFmtMxfp4;  // CacheFormat of the index, K and V pools
  float k_scale = 1.f;  // fp8 K tensor scale (1 for MXFP4)
  float v_scale = 1.f;  // fp8 V tensor scale (1 for MXFP4)
  const uint16_t* index_q;
  const uint8_t* index_pages;
  const uint16_t* q;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  int64_t num_pages;
  const int32_t* block_table;
  int bt_stride;
  const int32_t* seq_lens;
  int32_t* sel;        // selection: written by the index items, read by sparse attention
  float* sel_scores;   // nullable
  float scale;
  uint16_t* out;
  uint8_t* ws;
};
int launch_step(const StepArgs& a, const StepLayout& lay, hipStream_t stream, const char* what);

// The allocation-free step call's static scratch (step.hip): its size, and
// its address on the current device, set up on the first call per device
// (zeroed header; the stream is synchronised once).  Refused while the
// stream is being captured.
constexpr size_t kNoAllocScratchBytes = MONO_NOALLOC_SCRATCH_BYTES;
int noalloc_scratch(hipStream_t stream, uint8_t** ptr);
// Moves the error bits of the scratch's error word (at err_offset) into *dst.
int launch_scratch_errors(uint8_t* scratch_ptr, size_t err_offset, uint32_t* dst, hipStream_t stream);

}  // namespace mono
