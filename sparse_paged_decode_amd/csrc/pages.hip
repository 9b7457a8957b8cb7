// MXFP4 page packing, unpacking and dequantisation kernels (gfx950).
//
// Layout: page "vllm.models.minimax_m3.amd.ops.mxfp4_pages", module docstring
// -- 128 rows of 64 B e2m1 data (even element in the low nibble), then 128
// rows of 4 e8m0 scale bytes (one per 32 elements), 8704 B per page.
#include "device_common.h"
#include "launch.h"

namespace mono {
namespace {

// One thread per (page, row): 128 codes in, 64 data bytes + 4 scale bytes out.
__global__ __launch_bounds__(128) void pack_kernel(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales,
                                                   uint8_t* __restrict__ pages, int64_t n_rows) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= n_rows) return;
  const int64_t page = row / kPageTokens;
  const int r = (int)(row % kPageTokens);
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(codes + row * kHeadDim);
  uint8_t* dst_page = pages + page * kPageBytes;
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(dst_page + r * kRowBytes);
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // 32 codes -> 16 bytes
    u32x4_t a = src[2 * q], b = src[2 * q + 1];
    uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    u32x4_t out;
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      // dword w[2o] holds codes 8*(..)+0..3, w[2o+1] codes +4..7 (one per byte)
      uint32_t lo = w[2 * o], hi = w[2 * o + 1];
      uint32_t b0 = (lo & 0xFu) | ((lo >> 4) & 0xF0u);                     // codes 0,1
      uint32_t b1 = ((lo >> 16) & 0xFu) | ((lo >> 20) & 0xF0u);            // codes 2,3
      uint32_t b2 = (hi & 0xFu) | ((hi >> 4) & 0xF0u);                     // codes 4,5
      uint32_t b3 = ((hi >> 16) & 0xFu) | ((hi >> 20) & 0xF0u);            // codes 6,7
      out[o] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    }
    dst[q] = out;
  }
  const uint32_t s = *reinterpret_cast<const uint32_t*>(scales + row * 4);
  *reinterpret_cast<uint32_t*>(dst_page + kScaleOffset + r * 4) = s;
}

__global__ __launch_bounds__(128) void unpack_kernel(const uint8_t* __restrict__ pages,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales, int64_t n_rows) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= n_rows) return;
  const int64_t page = row / kPageTokens;
  const int r = (int)(row % kPageTokens);
  const uint8_t* src_page = pages + page * kPageBytes;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(src_page + r * kRowBytes);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + row * kHeadDim);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    u32x4_t in = src[q];
    u32x4_t a, b;
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      const uint32_t x = in[o];  // 4 bytes = 8 codes, even code in each low nibble
      const uint32_t c_lo = (x & 0xFu) | (((x >> 4) & 0xFu) << 8) | (((x >> 8) & 0xFu) << 16) |
                            (((x >> 12) & 0xFu) << 24);
      const uint32_t c_hi = ((x >> 16) & 0xFu) | (((x >> 20) & 0xFu) << 8) |
                            (((x >> 24) & 0xFu) << 16) | (((x >> 28) & 0xFu) << 24);
      if (o < 2) {
        a[2 * o] = c_lo;
        a[2 * o + 1] = c_hi;
      } else {
        b[2 * (o - 2)] = c_lo;
        b[2 * (o - 2) + 1] = c_hi;
      }
    }
    dst[2 * q] = a;
    dst[2 * q + 1] = b;
  }
  *reinterpret_cast<uint32_t*>(scales + row * 4) =
      *reinterpret_cast<const uint32_t*>(src_page + kScaleOffset + r * 4);
}

// One thread per (page, row, 32-element block).
__global__ __launch_bounds__(256) void dequant_f32_kernel(const uint8_t* __restrict__ pages,
                                                          float* __restrict__ out, int64_t n_blocks) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  const int64_t row = blk >> 2;
  const int g = (int)(blk & 3);
  const int64_t page = row / kPageTokens;
  const int r = (int)(row % kPageTokens);
  const uint8_t* p = pages + page * kPageBytes;
  const u32x4_t d = *reinterpret_cast<const u32x4_t*>(p + r * kRowBytes + 16 * g);
  const uint32_t e = p[kScaleOffset + r * 4 + g];
  f32x4_t* dst = reinterpret_cast<f32x4_t*>(out + row * kHeadDim + 32 * g);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f32x4_t v0, v1;
#pragma unroll
    for (int n = 0; n < 4; ++n) v0[n] = e2m1_times_e8m0_exact((d[w] >> (4 * n)) & 0xFu, e);
#pragma unroll
    for (int n = 0; n < 4; ++n) v1[n] = e2m1_times_e8m0_exact((d[w] >> (16 + 4 * n)) & 0xFu, e);
    dst[2 * w] = v0;
    dst[2 * w + 1] = v1;
  }
}

__global__ __launch_bounds__(256) void dequant_bf16_kernel(const uint8_t* __restrict__ pages,
                                                           uint16_t* __restrict__ out, int64_t n_blocks) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  const int64_t row = blk >> 2;
  const int g = (int)(blk & 3);
  const int64_t page = row / kPageTokens;
  const int r = (int)(row % kPageTokens);
  const uint8_t* p = pages + page * kPageBytes;
  const u32x4_t d = *reinterpret_cast<const u32x4_t*>(p + r * kRowBytes + 16 * g);
  const float scale = e8m0_scale_operand(p[kScaleOffset + r * 4 + g]);
  bf16x8_t* dst = reinterpret_cast<bf16x8_t*>(out + row * kHeadDim + 32 * g);
#pragma unroll
  for (int w = 0; w < 4; ++w) dst[w] = dequant8_bf16(d[w], scale);
}

inline unsigned grid_for(int64_t n, int block) { return (unsigned)((n + block - 1) / block); }

}  // namespace

int launch_pack(const uint8_t* codes, const uint8_t* scales, uint8_t* pages, int64_t n_pages,
                hipStream_t stream) {
  const int64_t n_rows = n_pages * kPageTokens;
  MONO_LAUNCH(kKPack, pack_kernel, dim3(grid_for(n_rows, 128)), dim3(128), 0, stream, codes, scales,
                     pages, n_rows);
  return check_launch("mxfp4_pages_pack");
}

int launch_unpack(const uint8_t* pages, uint8_t* codes, uint8_t* scales, int64_t n_pages,
                  hipStream_t stream) {
  const int64_t n_rows = n_pages * kPageTokens;
  MONO_LAUNCH(kKUnpack, unpack_kernel, dim3(grid_for(n_rows, 128)), dim3(128), 0, stream, pages, codes,
                     scales, n_rows);
  return check_launch("mxfp4_pages_unpack");
}

int launch_dequant_f32(const uint8_t* pages, float* out, int64_t n_pages, hipStream_t stream) {
  const int64_t n_blocks = n_pages * kPageTokens * 4;
  MONO_LAUNCH(kKDequant, dequant_f32_kernel, dim3(grid_for(n_blocks, 256)), dim3(256), 0, stream, pages,
                     out, n_blocks);
  return check_launch("mxfp4_pages_dequant");
}

int launch_dequant_bf16(const uint8_t* pages, uint16_t* out, int64_t n_pages, hipStream_t stream) {
  const int64_t n_blocks = n_pages * kPageTokens * 4;
  MONO_LAUNCH(kKDequantBf16, dequant_bf16_kernel, dim3(grid_for(n_blocks, 256)), dim3(256), 0, stream, pages,
                     out, n_blocks);
  return check_launch("mxfp4_pages_dequant_bf16");
}

}  // namespace mono
