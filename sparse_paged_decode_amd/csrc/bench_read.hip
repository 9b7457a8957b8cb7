// Read-bandwidth references for the benchmark (gfx950): how fast this part
// reads the bytes the index scan reads, with nothing else to do.
//
// Page geometry (page "vllm.models.minimax_m3.amd.ops.mxfp4_pages", module
// docstring): 8704-B pages, 128 rows of 64 data bytes, then 128 rows of 4
// scale bytes.  Two access patterns over n_pages pages:
//   mode 0 (stream):      the bytes [0, n_pages * 8704) in address order,
//                         16 B per lane per load;
//   mode 1 (page gather): the pages page_ids[0..n_pages) (a block-table
//                         order), each read with the scan's lane pattern:
//                         wave w takes rows 32w..32w+31 as two 16-row
//                         tiles, lane (g, m) the 16 data bytes of chunk g of
//                         its row and that chunk's scale byte.
// Each workgroup reads a contiguous run of the work with kAhead loads in
// flight per lane, folds what it read into one word and stores it to
// sink[blockIdx.x] (so no load is dead code).  Loads carry the
// non-temporal hint, as the scan's do.
#include "device_common.h"
#include "launch.h"

namespace mono {
namespace {

constexpr int kReadBlock = 256;
constexpr int kAhead = 8;  // 16-B loads in flight per lane (stream), pages in flight (gather)

__global__ __launch_bounds__(kReadBlock) void read_stream_kernel(const uint8_t* base, size_t n_vec, size_t per_wg,
                                                                 uint32_t* sink) {
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(base);
  const size_t v0 = (size_t)blockIdx.x * per_wg;
  const size_t v1 = min(v0 + per_wg, n_vec);
  uint32_t acc = 0;
  for (size_t v = v0 + threadIdx.x; v < v1; v += (size_t)kReadBlock * kAhead) {
    u32x4_t x[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const size_t idx = min(v + (size_t)u * kReadBlock, v1 - 1);
      x[u] = __builtin_nontemporal_load(p + idx);
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
  }
  acc ^= __shfl_xor(acc, 1);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(kReadBlock) void read_gather_kernel(const uint8_t* pages, const int32_t* page_ids,
                                                                 int n_pages, int per_wg, uint32_t* sink) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, m = lane & 15;
  const int row0 = 32 * wave + m;
  const uint32_t d0 = (uint32_t)(row0 * kRowBytes + 16 * g), d1 = d0 + 16 * kRowBytes;
  const uint32_t e0 = (uint32_t)(kScaleOffset + row0 * 4 + g), e1 = e0 + 16 * 4;
  const int p0 = blockIdx.x * per_wg, p1 = min(p0 + per_wg, n_pages);
  uint32_t acc = 0;
  for (int pb = p0; pb < p1; pb += kAhead) {
    u32x4_t x[kAhead][2];
    uint32_t e[kAhead][2];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const uint8_t* pg = pages + (size_t)page_ids[min(pb + u, p1 - 1)] * kPageBytes;
      x[u][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pg + d0));
      x[u][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pg + d1));
      e[u][0] = __builtin_nontemporal_load(pg + e0);
      e[u][1] = __builtin_nontemporal_load(pg + e1);
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u)
      acc ^= x[u][0][0] ^ x[u][0][3] ^ x[u][1][1] ^ x[u][1][2] ^ e[u][0] ^ (e[u][1] << 8);
  }
  acc ^= __shfl_xor(acc, 1);
  if (tid == 0) sink[blockIdx.x] = acc;
}

}  // namespace

int launch_read_reference(const uint8_t* pages, const int32_t* page_ids, int64_t n_pages, int mode, int grid,
                          uint32_t* sink, hipStream_t stream) {
  if (mode == 0) {
    const size_t n_vec = (size_t)n_pages * kPageBytes / 16;
    const size_t per_wg = (n_vec + grid - 1) / grid;
    MONO_LAUNCH(kKReadStream, read_stream_kernel, dim3(grid), dim3(kReadBlock), 0, stream, pages, n_vec, per_wg,
                sink);
  } else {
    const int per_wg = (int)((n_pages + grid - 1) / grid);
    MONO_LAUNCH(kKReadGather, read_gather_kernel, dim3(grid), dim3(kReadBlock), 0, stream, pages, page_ids,
                (int)n_pages, per_wg, sink);
  }
  return check_launch("mono_bench_read");
}

}  // namespace mono
