// Cache page formats the step kernel reads (gfx950).
//
// The scan and attention code is written once over a format policy that
// says how one lane fetches and converts its share of a row:
//   * a chunk: the 32 elements 32g..32g+31 of a row, converted for the
//     bf16 MFMA k-steps s = 0..3 (elements 32g + 8s .. 32g + 8s + 7);
//   * a slice: the 8 elements 8m..8m+7 of a row, converted to four bf16
//     pairs (elements 8m + 2p, 8m + 2p + 1), for the B operand of P V.
// Every conversion is exact in bf16.
#pragma once

#include "device_common.h"

namespace mono {

// MXFP4 (page "vllm.models.minimax_m3.amd.ops.mxfp4_pages", module
// docstring): 128 rows x 64 B of e2m1 (even element in the low nibble),
// then 128 rows x 4 B of e8m0 scales, one per 32 elements.
struct Mxfp4Format {
  static constexpr int kPageBytes = 8704;
  // Index pages a scan lane fetches ahead when the scores go to LDS (one
  // query row: the chunk-local step and the one-row scan items): two pages
  // ahead measured faster than one, three or four.
  static constexpr int kScanBatchLocal = 2;
  // The four-token instance (each page scored for up to four query tokens,
  // the scores staged in LDS): two pages ahead measured faster than three.
  static constexpr int kScanBatchMulti = 2;

  struct ChunkAddr {
    uint32_t d, e;  // byte offsets of the 16 data bytes and of the scale byte
  };
  struct Chunk {
    u32x4_t d;
    uint32_t e;
  };
  __device__ static ChunkAddr chunk_addr(int row, int g) {
    return {(uint32_t)(row * kRowBytes + 16 * g), (uint32_t)(kScaleOffset + row * 4 + g)};
  }
  __device__ static Chunk load_chunk(const uint8_t* page, ChunkAddr o) {
    return {*reinterpret_cast<const u32x4_t*>(page + o.d), page[o.e]};
  }
  // As load_chunk, for the index scan, which reads each page once: the loads
  // carry the non-temporal (streaming) hint.
  __device__ static Chunk load_chunk_stream(const uint8_t* page, ChunkAddr o) {
    return {__builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(page + o.d)),
            __builtin_nontemporal_load(page + o.e)};
  }
  __device__ static Chunk zero_chunk() { return {u32x4_t{0u, 0u, 0u, 0u}, 127u}; }
  __device__ static bf16x8_t chunk_bf16(const Chunk& c, int s) {
    return dequant8_bf16(c.d[s], e8m0_scale_operand(c.e));
  }

  struct Slice {
    uint32_t d, e;  // 4 data bytes (8 codes) and the scale of their block
  };
  __device__ static Slice load_slice(const uint8_t* page, uint32_t row, int m) {
    return {*reinterpret_cast<const uint32_t*>(page + row * kRowBytes + 4 * m), page[kScaleOffset + row * 4 + (m >> 2)]};
  }
  __device__ static Slice zero_slice() { return {0u, 127u}; }
  __device__ static u32x4_t slice_bf16(const Slice& v) {
    return __builtin_bit_cast(u32x4_t, dequant8_bf16(v.d, e8m0_scale_operand(v.e)));
  }
};

// fp8 (the older build's caches: weights page SparseMoeLayer, "fp8" index
// cache; dispatch page _config_refusal, fp8 KV cache): 128 rows x 128 B of
// OCP e4m3, element i of row r at byte 128r + i.  A per-tensor K or V scale
// is applied outside, to the logits and to the output.
struct Fp8Format {
  static constexpr int kPageBytes = 16384;
  static constexpr int kRowBytes8 = 128;
  static constexpr int kScanBatchLocal = 2;  // one page ahead measured slower
  static constexpr int kScanBatchMulti = 2;

  struct ChunkAddr {
    uint32_t d;
  };
  struct Chunk {
    u32x4_t d[2];  // elements 32g..32g+15, 32g+16..32g+31
  };
  __device__ static ChunkAddr chunk_addr(int row, int g) { return {(uint32_t)(row * kRowBytes8 + 32 * g)}; }
  __device__ static Chunk load_chunk(const uint8_t* page, ChunkAddr o) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(page + o.d);
    return {{p[0], p[1]}};
  }
  // The index scan's loads: plain here (the streaming hint made the fp8 scan
  // slower, where it speeds up the MXFP4 one).
  __device__ static Chunk load_chunk_stream(const uint8_t* page, ChunkAddr o) { return load_chunk(page, o); }
  __device__ static Chunk zero_chunk() { return {{u32x4_t{0u, 0u, 0u, 0u}, u32x4_t{0u, 0u, 0u, 0u}}}; }
  // Four e4m3 bytes of one dword -> bf16 pairs (bytes 0,1) and (bytes 2,3).
  __device__ static uint32_t pair_lo(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  }
  __device__ static uint32_t pair_hi(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  }
  __device__ static bf16x8_t chunk_bf16(const Chunk& c, int s) {
    const uint32_t w0 = c.d[s >> 1][(2 * s) & 3], w1 = c.d[s >> 1][(2 * s + 1) & 3];
    return __builtin_bit_cast(bf16x8_t, u32x4_t{pair_lo(w0), pair_hi(w0), pair_lo(w1), pair_hi(w1)});
  }

  struct Slice {
    uint32_t d0, d1;  // elements 8m..8m+3, 8m+4..8m+7
  };
  __device__ static Slice load_slice(const uint8_t* page, uint32_t row, int m) {
    const uint2 v = *reinterpret_cast<const uint2*>(page + row * kRowBytes8 + 8 * m);
    return {v.x, v.y};
  }
  __device__ static Slice zero_slice() { return {0u, 0u}; }
  __device__ static u32x4_t slice_bf16(const Slice& v) {
    return u32x4_t{pair_lo(v.d0), pair_hi(v.d0), pair_lo(v.d1), pair_hi(v.d1)};
  }
};

}  // namespace mono
