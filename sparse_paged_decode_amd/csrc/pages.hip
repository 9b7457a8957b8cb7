// MXFP4 page packing, unpacking and dequantisation kernels (gfx950).
//
// Layout: page "vllm.models.minimax_m3.amd.ops.mxfp4_pages", module docstring
// -- 128 rows of 64 B e2m1 data (even element in the low nibble), then 128
// rows of 4 e8m0 scale bytes (one per 32 elements), 8704 B per page.
#include "device_common.h"
#include "launch.h"
#include "page_format.h"

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

// fp8 pages: one thread per (page, row, 32-element chunk), converted by the
// step kernel's own chunk conversion.
__global__ __launch_bounds__(256) void dequant_fp8_bf16_kernel(const uint8_t* __restrict__ pages,
                                                               uint16_t* __restrict__ out, int64_t n_chunks) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n_chunks) return;
  const int64_t row = c >> 2;
  const int g = (int)(c & 3);
  const uint8_t* p = pages + (row / kPageTokens) * Fp8Format::kPageBytes;
  const Fp8Format::Chunk ch = Fp8Format::load_chunk(p, Fp8Format::chunk_addr((int)(row % kPageTokens), g));
  bf16x8_t* dst = reinterpret_cast<bf16x8_t*>(out + row * kHeadDim + 32 * g);
#pragma unroll
  for (int s = 0; s < 4; ++s) dst[s] = Fp8Format::chunk_bf16(ch, s);
}

// ---- the cache insert ---------------------------------------------------------
// Rounding rule (OCP Microscaling v1.0 conversion; the pages name the writer
// but not its rule): per 32-element block the scale byte is
// floor(log2 max|v|) - 2 + 127 clamped to [0, 254]; each element goes to the
// nearest e2m1 magnitude of v / 2^(byte-127), ties to the even code, above
// 6 saturating; NaN or +-inf anywhere gives byte 0xFF and codes 0; an
// all-zero block gives byte 0.
//
// The element codes come from v_cvt_scalef32_pk_fp4_f32 with the block's
// e8m0 scale 2^(byte-127): it converts two fp32 values (each bf16 exactly)
// to e2m1 codes of value / scale, nearest with ties to the even code,
// saturating at 6, keeping the sign (-0.0 gives code 8), and packs them
// into one byte, the first in the low nibble.  That is the conversion
// above; it was checked for every positive finite bf16 value at every scale
// byte that keeps the quotient below 8, both signs, against the
// nearest-with-ties-to-even rule.
struct InsertArgs {
  const uint16_t* rows[3];  // K [n, heads, 128], V [n, heads, 128], index key [n, 128] (bf16 bits)
  uint8_t* pools[3];        // [num_pages, heads, 8704] x 2, [num_pages, 8704]
  int row_heads[3];         // rows per token of each cache (0: not written)
  int64_t row_end[3];       // running sums of n * row_heads: cache c owns rows [row_end[c-1], row_end[c])
  const int64_t* slots;     // [n]
  int64_t n_threads;        // 4 * row_end[2]
  int64_t num_pages;
  uint32_t* err;
};

// One thread per (cache row, 32-element block): reads the block's 64 B of
// bf16, writes its 16 B of packed e2m1 and its scale byte.  Rows are ordered
// cache-major, then token, then head, so the four threads of a row are
// adjacent lanes and a wave covers consecutive rows of one cache: its reads,
// its data writes and its scale writes are each contiguous runs when the
// slots are consecutive.
__global__ __launch_bounds__(256) void insert_kernel(InsertArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= a.n_threads) return;
  const int blk = (int)(tid & 3);
  const int64_t row = tid >> 2;
  const int c = (row >= a.row_end[0]) + (row >= a.row_end[1]);
  const int64_t local = row - (c ? a.row_end[c - 1] : 0);  // = t * heads + j
  const int heads = a.row_heads[c];
  const int64_t t = local / heads;
  const int j = (int)(local - t * heads);
  // The row is loaded before the slot is looked at, so the two loads overlap.
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.rows[c] + local * kHeadDim + blk * kScaleBlock);
  u32x4_t in[4];
#pragma unroll
  for (int L = 0; L < 4; ++L) in[L] = src[L];
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  const int64_t page = slot >> 7;
  if (page >= a.num_pages) {
    if (blk == 0 && j == 0) raise_error(a.err, kErrSlot);
    return;
  }
  uint32_t amax = 0;
#pragma unroll
  for (int L = 0; L < 4; ++L)
#pragma unroll
    for (int d = 0; d < 4; ++d) amax = max(amax, max(in[L][d] & 0x7FFFu, (in[L][d] >> 16) & 0x7FFFu));
  int byte;
  if (amax >= 0x7F80u) {
    byte = 0xFF;
  } else if (amax == 0) {
    byte = 0;
  } else {
    const uint32_t E = amax >> 7;
    const int flog2 = E ? (int)E - 127 : -133 + (31 - (int)__builtin_clz(amax & 0x7Fu));
    byte = min(max(flog2 - 2 + 127, 0), 254);
  }
  const float scale = e8m0_scale_operand((uint32_t)byte);  // 2^(byte - 127)
  u32x4_t out;
#pragma unroll
  for (int L = 0; L < 4; ++L) {  // bf16 elements 8L..8L+7 -> codes in nibbles of word L
    // byte p of the word takes elements 8L+2p (low nibble) and 8L+2p+1
    auto lo = [&](int p) { return __uint_as_float(in[L][p] << 16); };
    auto hi = [&](int p) { return __uint_as_float(in[L][p] & 0xFFFF0000u); };
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, lo(0), hi(0), scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, lo(1), hi(1), scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, lo(2), hi(2), scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, lo(3), hi(3), scale, 3);
    out[L] = byte == 0xFF ? 0u : w;
  }
  const int r = (int)(slot & (kPageTokens - 1));
  uint8_t* pg = a.pools[c] + (page * heads + j) * kPageBytes;
  *reinterpret_cast<u32x4_t*>(pg + r * kRowBytes + 16 * blk) = out;
  pg[kScaleOffset + r * 4 + blk] = (uint8_t)byte;
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

int launch_dequant_fp8_bf16(const uint8_t* pages, uint16_t* out, int64_t n_pages, hipStream_t stream) {
  const int64_t n_chunks = n_pages * kPageTokens * 4;
  MONO_LAUNCH(kKDequantFp8Bf16, dequant_fp8_bf16_kernel, dim3(grid_for(n_chunks, 256)), dim3(256), 0, stream, pages,
              out, n_chunks);
  return check_launch("fp8_pages_dequant_bf16");
}

int launch_insert(const uint16_t* const rows[3], uint8_t* const pools[3], const int row_heads[3],
                  const int64_t* slots, int64_t n, int64_t num_pages, uint32_t* err, hipStream_t stream) {
  InsertArgs a{};
  int64_t end = 0;
  for (int c = 0; c < 3; ++c) {
    a.rows[c] = rows[c];
    a.pools[c] = pools[c];
    a.row_heads[c] = row_heads[c];
    end += n * row_heads[c];
    a.row_end[c] = end;
  }
  a.slots = slots;
  a.n_threads = 4 * end;
  a.num_pages = num_pages;
  a.err = err;
  MONO_LAUNCH(kKInsert, insert_kernel, dim3(grid_for(a.n_threads, 256)), dim3(256), 0, stream, a);
  return check_launch("mono_insert_mxfp4");
}

}  // namespace mono
