// Device helpers shared by the gfx950 kernels of libmono_decode.so.
//
// Page layout (page "vllm.models.minimax_m3.amd.ops.mxfp4_pages", module
// docstring): a page is 128 rows of 64 B packed e2m1 data (element 2c in the
// low nibble of byte c, element 2c+1 in the high nibble) followed by 128 rows
// of 4 e8m0 scale bytes, one per 32 elements; 8704 B, no global scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"
#include "trace.h"

namespace mono {

constexpr int kRowBytes = 64;        // packed e2m1 bytes per row
constexpr int kScaleBlock = 32;      // elements per e8m0 scale
constexpr int kScaleOffset = 8192;   // 128 rows x 64 B
constexpr int kPageBytes = 8704;     // + 128 rows x 4 B

// Workspace error word bits (mirrors MONO_DEVERR_* of the public header).
constexpr uint32_t kErrPageId = 1u;
constexpr uint32_t kErrSeqLen = 2u;
constexpr uint32_t kErrSelection = 4u;  // selection counts inconsistent (never expected)
constexpr uint32_t kErrWait = 8u;       // a bounded wait for another work item ran out
constexpr uint32_t kErrSlot = 16u;      // an insert slot past the pool

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// e8m0 byte -> the fp32 scale operand of the gfx950 scaled fp4 conversions:
// the byte in the operand's exponent field, zero mantissa.  The conversions
// read only that field as the e8m0 scale, so bytes 0 (2^-127) and 255 (NaN)
// need no special case (checked bit for bit on all 16 codes x 256 bytes).
__device__ __forceinline__ float e8m0_scale_operand(uint32_t e) { return __uint_as_float(e << 23); }

// Eight e2m1 codes (one dword of packed row data: elements 8w..8w+7 when the
// dword is the w-th of the row) -> eight bf16 values times the block scale,
// in element order.  v_cvt_scalef32_pk_bf16_fp4 converts the two nibbles of
// one selected byte; bf16 has fp32's exponent range, so every finite
// product of an e2m1 value and an e8m0 scale is exact.
__device__ __forceinline__ bf16x8_t dequant8_bf16(uint32_t packed, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 3);
  bf16x8_t r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

// Exact fp32 value of one e2m1 code times 2^(e-127), built from integer
// fields: code magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 are m * 2^-1 with
// m = 0, 1, 2, 3, 4, 6, 8, 12; ldexp then applies the scale with IEEE
// rounding (subnormal results stay exact, overflow gives inf).
__device__ __forceinline__ float e2m1_times_e8m0_exact(uint32_t code, uint32_t e) {
  const uint32_t mag_half = (0xC8643210u >> (4u * (code & 7u))) & 0xFu;  // m above
  float v = (float)mag_half;
  v = (code & 8u) ? -v : v;
  if (e == 255u) return __uint_as_float(0x7fc00000u);
  // 2^(e-127) * m / 2 in two steps so no intermediate leaves the range early.
  return __builtin_amdgcn_ldexpf(v, (int)e - 128);
}

// Monotone fp32 -> uint32 key: a > b as floats <=> key(a) > key(b); NaN maps
// to 0, below every number.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (s != s) ? 0u : k;
}

__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// threadIdx.x read through an empty asm statement.  Values derived from it
// then cannot be hoisted out of the persistent kernel's work-item loop,
// where they would stay live across every kind of item and crowd out the
// registers each item needs.
__device__ __forceinline__ int thread_index() {
  int t = __builtin_amdgcn_workitem_id_x();
  asm volatile("" : "+v"(t));
  return t;
}

// Set device error bits in the workspace error word.
__device__ __forceinline__ void raise_error(uint32_t* err, uint32_t bits) {
  atomicOr(err, bits);
}

// Cross-workgroup hand-off within one kernel.  On gfx950 an agent-scope
// fence writes back and invalidates the whole L2 of the XCD, which costs far
// more than the data it protects.  Instead, every value one workgroup hands
// to another is written and read with agent-scope atomic stores/loads (these
// are coherent across XCDs by themselves), and the producer waits for its
// memory operations to complete (vmcnt 0) before a barrier and the counter
// increment that publishes them.
__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_coherent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes per lane written with the same agent-scope coherence (the sc1
// policy), through a raw buffer resource over [base, base + bytes) whose
// out-of-range offsets the hardware drops.  For hand-offs of whole blocks:
// with lane-contiguous offsets a wave writes full 64-B lines.
constexpr int kBufferFormatWord = 0x00020000;  // dword 3 of a raw gfx9 buffer resource
constexpr int kPolicyAgentCoherent = 16;       // the sc1 bit of the cache-policy operand
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFormatWord);
}
__device__ __forceinline__ void store_coherent_x4(__amdgpu_buffer_rsrc_t r, uint32_t offset, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)offset, 0, kPolicyAgentCoherent);
}
// 16 bytes per lane read with the same agent-scope coherence as
// load_coherent (the sc1 policy); offsets past the resource read zero.
__device__ __forceinline__ u32x4_t load_coherent_x4(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)offset, 0, kPolicyAgentCoherent);
}
// Wait until this thread's outstanding vector memory operations (loads,
// stores, atomics) have completed; also a compiler memory barrier.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace mono
