// Paged GQA decode attention over MXFP4 K/V pages (gfx950).
//
// The pa_decode the mxfp4_pages page names reads [pages, heads, 8704] K and V
// pools as [pages, heads, 128, 64] data and [pages, heads, 128, 4] scales
// (page "vllm.models.minimax_m3.amd.ops.mxfp4_pages", mxfp4_page_views).
// Per query token: logits scale * q_h . k_j for the 16 query heads of a KV
// head over the candidate tokens (a selection list, or every token
// 0..pos), softmax, and the probability-weighted sum of the V rows.
//
// Work split: one workgroup per (query token, split of `split_tokens`
// candidates, KV head); each wave takes groups of 32 candidates.  Per group:
//   * QK^T on bf16 MFMA 16x16x32 with the *tokens* as the M dimension (two
//     16-token tiles) and the 16 query heads as N, so each lane ends with the
//     logits of one head for 8 tokens -- exactly the B-operand layout the PV
//     product needs for the probabilities;
//   * online softmax in the log2 domain (running max and sum per head);
//   * PV as O^T = V^T P^T on the same MFMA: V is dequantised to bf16 and
//     written transposed into LDS (dims x token pairs), then read back 8
//     tokens per lane with one 16-byte LDS load per 16-dim tile.
// Dequantised K/V are exact in bf16, so the only roundings are fp32
// accumulation, exp2, and the bf16 rounding of the probabilities (the row
// sums use the same rounded values).  Workgroup partials (max, sum, 16x128
// accumulator) are merged by the last workgroup of each (query, KV head).
#include "block_ops.h"
#include "launch.h"

namespace mono {

constexpr int kGroupTokens = 32;
constexpr int kVtRowBytes = 80;        // 16 token pairs x 4 B + 16 B pad
constexpr int kVtRegionBytes = 10496;  // 128 rows + 3 x 64 B group pad, per wave

PaLayout pa_layout(int B, int T, int kv_heads, int bt_stride, int k, int sparse) {
  PaLayout l{};
  const size_t NH = (size_t)B * T * kv_heads;
  const long list_max = sparse ? (long)k : (long)bt_stride * kPageTokens;
  int split = 256;
  while (split < 8192 && NH * (size_t)((list_max + split - 1) / split) > 4096) split *= 2;
  l.split_tokens = split;
  l.n_splits = (int)((list_max + split - 1) / split);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t S = (size_t)l.n_splits;
  l.err = take(256);
  l.cnt = take(NH * 4);
  l.pm = take(NH * S * kQHeads * 4);
  l.pl = take(NH * S * kQHeads * 4);
  l.pacc = take(NH * S * kQHeads * kHeadDim * 4);
  l.total = off;
  return l;
}

namespace {

__device__ __forceinline__ int vt_offset(int dim, int pair) {
  return dim * kVtRowBytes + (dim >> 5) * 64 + pair * 4;
}

__device__ __forceinline__ void store_bf16x8(uint16_t* dst, const float* o, float inv) {
  u32x4_t w;
#pragma unroll
  for (int x = 0; x < 4; ++x) w[x] = bf16x2_bits(o[2 * x] * inv, o[2 * x + 1] * inv);
  *reinterpret_cast<u32x4_t*>(dst) = w;
}

// grid (B*T, splits, kv_heads); 256 threads.
template <bool SPARSE>
__global__ __launch_bounds__(256) void pa_decode_kernel(PaArgs a, PaLayout lay) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * kVtRegionBytes];
  __shared__ float s_m[kWaves][kQHeads];
  __shared__ float s_l[kWaves][kQHeads];
  __shared__ uint32_t s_last;

  const int i = blockIdx.x, split = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, m = lane & 15;
  uint32_t* err = reinterpret_cast<uint32_t*>(a.ws + lay.err);
  const int b = i / a.T, t = i % a.T;
  const int L = a.seq_lens[b];
  if (L < a.T || L > a.bt_stride * kPageTokens) {
    if (split == 0 && h == 0 && tid == 0) raise_error(err, kErrSeqLen);
    return;
  }
  const int pos = L - a.T + t;
  const int list_len = SPARSE ? a.k : pos + 1;
  const int n_splits = SPARSE ? lay.n_splits : (list_len + lay.split_tokens - 1) / lay.split_tokens;
  if (split >= n_splits) return;
  const int e0 = split * lay.split_tokens;
  const int e1 = min(e0 + lay.split_tokens, list_len);
  const int n_groups = (e1 - e0 + kGroupTokens - 1) / kGroupTokens;
  const int iters = (n_groups + kWaves - 1) / kWaves;
  const int H = a.kv_heads;

  // B operand of QK^T: column n = m is query head 16h + m; k-slot (g, e) of
  // k-step s holds q element 32g + 8s + e.
  bf16x8_t qb[4];
  {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        a.q + ((size_t)i * H * kQHeads + (size_t)h * kQHeads + m) * kHeadDim + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = __builtin_bit_cast(bf16x8_t, src[s]);
  }
  const float sl2 = a.scale * 1.4426950408889634f;  // logits in log2 units
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t acc[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) acc[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint8_t* vt = lds + wave * kVtRegionBytes;
  const int32_t* sel_row = SPARSE ? a.selected_idx + (size_t)i * a.k : nullptr;
  const int32_t* bt_row = a.block_table + (size_t)b * a.bt_stride;

  // Groups are processed two at a time; the token lookups, block-table
  // lookups and K/V loads of both are issued before either is computed, so
  // each stage costs one memory round trip for the pair.
  struct Tok {
    u32x4_t kd, vd;
    uint32_t ke, ve;
    bool valid;
  };
  for (int it0 = 0; it0 < iters; it0 += 2) {
    Tok tk[2][2];
    int jj[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // lane (g, m) handles tokens 2m and 2m+1 of each 32-token group
        const int entry = e0 + kGroupTokens * (wave + kWaves * (it0 + x)) + 2 * m + u;
        int j = -1;
        if (it0 + x < iters && entry < e1) j = SPARSE ? sel_row[entry] : entry;
        jj[x][u] = (j >= 0 && j <= pos) ? j : -1;
      }
    int pid[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int u = 0; u < 2; ++u) pid[x][u] = jj[x][u] >= 0 ? bt_row[jj[x][u] >> 7] : -1;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        Tok& t = tk[x][u];
        t.kd = t.vd = u32x4_t{0u, 0u, 0u, 0u};
        t.ke = t.ve = 127u;
        t.valid = false;
        const int j = jj[x][u];
        if (j >= 0) {
          if (pid[x][u] < 0 || pid[x][u] >= a.num_pages) {
            raise_error(err, kErrPageId);
          } else {
            const size_t off = ((size_t)pid[x][u] * H + h) * kPageBytes;
            const int r = j & (kPageTokens - 1);
            t.kd = *reinterpret_cast<const u32x4_t*>(a.k_pages + off + r * kRowBytes + 16 * g);
            t.vd = *reinterpret_cast<const u32x4_t*>(a.v_pages + off + r * kRowBytes + 16 * g);
            t.ke = a.k_pages[off + kScaleOffset + r * 4 + g];
            t.ve = a.v_pages[off + kScaleOffset + r * 4 + g];
            t.valid = true;
          }
        }
      }
#pragma unroll
  for (int xi = 0; xi < 2; ++xi) {
    if (it0 + xi >= iters) break;  // uniform across the workgroup
    u32x4_t kd[2] = {tk[xi][0].kd, tk[xi][1].kd}, vd[2] = {tk[xi][0].vd, tk[xi][1].vd};
    uint32_t ke[2] = {tk[xi][0].ke, tk[xi][1].ke}, ve[2] = {tk[xi][0].ve, tk[xi][1].ve};
    bool valid[2] = {tk[xi][0].valid, tk[xi][1].valid};

    // S^T tiles: lane (g, n) gets tokens 8g + 2i + u (i = 0..3) of head n.
    f32x4_t c[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float sc = e8m0_scale_operand(ke[u]);
      c[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        c[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8_bf16(kd[u][s], sc), qb[s], c[u], 0, 0, 0);
    }
    // Validity of token 2r + u sits in bit r of these ballots (lanes 0..15).
    const uint32_t vm0 = (uint32_t)__ballot(valid[0]);
    const uint32_t vm1 = (uint32_t)__ballot(valid[1]);
    float z[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t vm = u ? vm1 : vm0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool v = (vm >> (4 * g + r)) & 1u;
        z[u][r] = v ? c[u][r] * sl2 : -INFINITY;
        mx = fmaxf(mx, z[u][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    u32x4_t pw;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pw[r] = bf16x2_bits(__builtin_amdgcn_exp2f(z[0][r] - m_use), __builtin_amdgcn_exp2f(z[1][r] - m_use));
      psum += bf16_lo_to_f32(pw[r]) + bf16_hi_to_f32(pw[r]);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] *= alpha;
    // k-slot (g, e) of P^T is token 8g + e, e = 2r + u.
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);

    // V^T into LDS: row = dim, column = token pair m (tokens 2m, 2m+1).
    {
      const float sv0 = e8m0_scale_operand(ve[0]);
      const float sv1 = e8m0_scale_operand(ve[1]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4_t w0 = __builtin_bit_cast(u32x4_t, dequant8_bf16(vd[0][s], sv0));
        const u32x4_t w1 = __builtin_bit_cast(u32x4_t, dequant8_bf16(vd[1][s], sv1));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int d = 32 * g + 8 * s + 2 * q;
          *reinterpret_cast<uint32_t*>(vt + vt_offset(d, m)) = (w0[q] & 0xffffu) | (w1[q] << 16);
          *reinterpret_cast<uint32_t*>(vt + vt_offset(d + 1, m)) = (w0[q] >> 16) | (w1[q] & 0xffff0000u);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      // A operand: row m is dim 16x + m, k-slot (g, e) is token 8g + e.
      const bf16x8_t va =
          __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(vt + vt_offset(16 * x + m, 4 * g)));
      acc[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[x], 0, 0, 0);
    }
    __syncthreads();
  }
  }

  // ---- combine the four waves -------------------------------------------
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  float* so = reinterpret_cast<float*>(lds);  // [wave][dim][head], 8 KiB per wave
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) so[wave * 2048 + (16 * x + 4 * g + r) * kQHeads + m] = acc[x][r];
  if (g == 0) {
    s_m[wave][m] = m_run;
    s_l[wave][m] = l_run;
  }
  __syncthreads();
  const int hd = tid >> 4;         // query head within the group
  const int d0 = (tid & 15) * 8;   // first of this thread's 8 dims
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][hd]);
  float Mu = (M == -INFINITY) ? 0.f : M;
  float lsum = 0.f, o[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) o[x] = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float f = __builtin_amdgcn_exp2f(s_m[w][hd] - Mu);
    lsum += s_l[w][hd] * f;
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] += so[w * 2048 + (d0 + x) * kQHeads + hd] * f;
  }

  const size_t qh = (size_t)i * H + h;
  uint16_t* orow = a.out + (qh * kQHeads + hd) * kHeadDim + d0;
  if (n_splits == 1) {
    store_bf16x8(orow, o, lsum > 0.f ? 1.f / lsum : 0.f);
    return;
  }

  const size_t slot = qh * lay.n_splits + split;
  float* pm = reinterpret_cast<float*>(a.ws + lay.pm);
  float* pl = reinterpret_cast<float*>(a.ws + lay.pl);
  float* pacc = reinterpret_cast<float*>(a.ws + lay.pacc);
  if ((tid & 15) == 0) {
    store_coherent(pm + slot * kQHeads + hd, M);
    store_coherent(pl + slot * kQHeads + hd, lsum);
  }
  {
    float* dst = pacc + (slot * kQHeads + hd) * kHeadDim + d0;
#pragma unroll
    for (int x = 0; x < 8; ++x) store_coherent(dst + x, o[x]);
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    uint32_t* cnt = reinterpret_cast<uint32_t*>(a.ws + lay.cnt) + qh;
    const uint32_t prev = atomicAdd(cnt, 1u);
    s_last = (prev == (uint32_t)(n_splits - 1)) ? 1u : 0u;
    if (s_last) *cnt = 0u;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- last workgroup: merge the splits of this (query token, KV head) ----
  // (partials are read with coherent loads)
  // Splits are read four at a time so their loads overlap.
  const size_t s0 = qh * lay.n_splits;
  M = -INFINITY;
  for (int s = 0; s < n_splits; s += 4) {
    float mv[4];
#pragma unroll
    for (int y = 0; y < 4; ++y) mv[y] = (s + y < n_splits) ? load_coherent(pm + (s0 + s + y) * kQHeads + hd) : -INFINITY;
#pragma unroll
    for (int y = 0; y < 4; ++y) M = fmaxf(M, mv[y]);
  }
  Mu = (M == -INFINITY) ? 0.f : M;
  lsum = 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x) o[x] = 0.f;
  for (int s = 0; s < n_splits; s += 4) {
    float mv[4], lv[4], av[4][8];
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const bool in = s + y < n_splits;
      const size_t sl = s0 + s + (in ? y : 0);
      mv[y] = in ? load_coherent(pm + sl * kQHeads + hd) : -INFINITY;
      lv[y] = in ? load_coherent(pl + sl * kQHeads + hd) : 0.f;
      const float* src = pacc + (sl * kQHeads + hd) * kHeadDim + d0;
#pragma unroll
      for (int x = 0; x < 8; ++x) av[y][x] = in ? load_coherent(src + x) : 0.f;
    }
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const float f = __builtin_amdgcn_exp2f(mv[y] - Mu);
      lsum += lv[y] * f;
#pragma unroll
      for (int x = 0; x < 8; ++x) o[x] += av[y][x] * f;
    }
  }
  store_bf16x8(orow, o, lsum > 0.f ? 1.f / lsum : 0.f);
}

}  // namespace

int launch_pa_decode(const PaArgs& a, const PaLayout& lay, hipStream_t stream) {
  const dim3 grid((unsigned)(a.B * a.T), (unsigned)lay.n_splits, (unsigned)a.kv_heads);
  if (a.selected_idx) {
    MONO_LAUNCH(kKPaDecode, pa_decode_kernel<true>, grid, dim3(kBlock), 0, stream, a, lay);
  } else {
    MONO_LAUNCH(kKPaDecode, pa_decode_kernel<false>, grid, dim3(kBlock), 0, stream, a, lay);
  }
  return check_launch("mono_pa_decode_mxfp4");
}

}  // namespace mono
