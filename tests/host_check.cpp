// Host-side checks of libmono_decode.so's argument validation and launch
// plan, built with g++ and the address and undefined-behaviour sanitizers
// from the library's own plan.cpp (no HIP runtime, no device).
//
// Every precondition of the C ABI (include/mono_decode.h) is driven into its
// error code; the workspace layouts and launch plans of the workloads' shapes
// and of random shapes are checked for the invariants the kernels rely on,
// among them that the chunk-local instance is refused whenever its chunk
// items would not all be resident at once.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <random>

#include "plan.h"

using namespace mono;

static int g_checks = 0, g_failures = 0;

#define CHECK(cond)                                                          \
  do {                                                                       \
    ++g_checks;                                                              \
    if (!(cond)) {                                                           \
      ++g_failures;                                                          \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);     \
    }                                                                        \
  } while (0)

// A code and a non-empty message; the message is cleared afterwards.
#define EXPECT_CODE(expr, code)                                              \
  do {                                                                       \
    clear_error();                                                           \
    const int rc_ = (expr);                                                  \
    CHECK(rc_ == (code));                                                    \
    if ((code) != MONO_OK) CHECK(strlen(last_error()) > 0);                  \
    if (rc_ != (code)) fprintf(stderr, "   got %d (%s)\n", rc_, last_error()); \
  } while (0)

// Distinct aligned stand-ins for device pointers (never dereferenced).
static const void* ptr(uintptr_t i) { return reinterpret_cast<const void*>((uintptr_t)0x100000 * (i + 1)); }
static const void* misaligned(uintptr_t i) { return reinterpret_cast<const void*>((uintptr_t)0x100000 * (i + 1) + 2); }

static void check_shapes() {
  EXPECT_CODE(check_step_shape(1, 1, 1, 1, true), MONO_OK);
  EXPECT_CODE(check_step_shape(0, 1, 1, 1, true), MONO_EINVAL);
  EXPECT_CODE(check_step_shape(1, 0, 1, 1, true), MONO_EINVAL);
  EXPECT_CODE(check_step_shape(1 << 20, 1 << 11, 1, 1, true), MONO_EINVAL);  // B*T > 2^30
  EXPECT_CODE(check_step_shape(1, 1, 0, 1, true), MONO_EINVAL);
  EXPECT_CODE(check_step_shape(1, 1, kMaxBtStride + 1, 1, true), MONO_EINVAL);
  EXPECT_CODE(check_step_shape(1, 1, 2, 0, true), MONO_EINVAL);
  EXPECT_CODE(check_step_shape(1, 1, 2, 257, true), MONO_EINVAL);  // k past 2 pages
  EXPECT_CODE(check_step_shape(1, 1, 2, 256, true), MONO_OK);
  EXPECT_CODE(check_step_shape(1, 1, 2, 0, false), MONO_OK);      // dense attention: k unused
}

static void check_pages() {
  EXPECT_CODE(check_pages_args(ptr(0), ptr(1), ptr(2), 3, 16, 4, 16, "pack"), MONO_OK);
  EXPECT_CODE(check_pages_args(nullptr, nullptr, nullptr, 0, 16, 4, 16, "pack"), MONO_OK);  // n = 0: no-op
  EXPECT_CODE(check_pages_args(ptr(0), ptr(1), ptr(2), -1, 16, 4, 16, "pack"), MONO_EINVAL);
  EXPECT_CODE(check_pages_args(ptr(0), ptr(1), ptr(2), ((int64_t)1 << 34) + 1, 16, 4, 16, "pack"), MONO_EINVAL);
  EXPECT_CODE(check_pages_args(nullptr, ptr(1), ptr(2), 1, 16, 4, 16, "pack"), MONO_EINVAL);
  EXPECT_CODE(check_pages_args(ptr(0), nullptr, ptr(2), 1, 16, 4, 16, "pack"), MONO_EINVAL);
  EXPECT_CODE(check_pages_args(ptr(0), ptr(1), nullptr, 1, 16, 4, 16, "pack"), MONO_EINVAL);
  EXPECT_CODE(check_pages_args(misaligned(0), ptr(1), ptr(2), 1, 16, 4, 16, "pack"), MONO_EINVAL);
  EXPECT_CODE(check_pages_args(ptr(0), misaligned(1), ptr(2), 1, 16, 4, 16, "pack"), MONO_EINVAL);
}

static void check_index() {
  StepLayout lay{};
  const size_t ws = (size_t)1 << 30;
  auto call = [&](const void* iq, const void* ip, int64_t np, const void* bt, int bts, const void* sl, int B, int T,
                  int k, const void* sel, const void* scores, const void* w, size_t wsb, int lo, int hi) {
    return check_index_call("index", iq, ip, np, bt, bts, sl, B, T, k, sel, scores, w, wsb, lo, hi, &lay);
  };
  EXPECT_CODE(call(ptr(0), ptr(1), 10, ptr(2), 4, ptr(3), 2, 1, 8, ptr(4), nullptr, ptr(5), ws, 0, -1), MONO_OK);
  CHECK(lay.total > 0 && lay.total <= ws && lay.win_lo == 0 && lay.win_hi == 4);
  const size_t need = lay.total;
  EXPECT_CODE(call(ptr(0), ptr(1), 10, ptr(2), 4, ptr(3), 2, 1, 8, ptr(4), nullptr, ptr(5), need - 1, 0, -1),
              MONO_ENOSPC);
  EXPECT_CODE(call(ptr(0), ptr(1), 10, ptr(2), 4, ptr(3), 2, 1, 8, ptr(4), nullptr, ptr(5), need, 0, -1), MONO_OK);
  EXPECT_CODE(call(ptr(0), ptr(1), 10, ptr(2), 4, ptr(3), 2, 1, 8, ptr(4), ptr(6), ptr(5), ws, 1, 3), MONO_OK);
  CHECK(lay.win_lo == 1 && lay.win_hi == 3);
  for (auto w : {std::pair<int, int>{-1, 2}, {2, 2}, {3, 2}, {0, 5}})
    EXPECT_CODE(call(ptr(0), ptr(1), 10, ptr(2), 4, ptr(3), 2, 1, 8, ptr(4), nullptr, ptr(5), ws, w.first, w.second),
                MONO_EINVAL);
  EXPECT_CODE(call(nullptr, ptr(1), 10, ptr(2), 4, ptr(3), 2, 1, 8, ptr(4), nullptr, ptr(5), ws, 0, -1), MONO_EINVAL);
  EXPECT_CODE(call(ptr(0), nullptr, 10, ptr(2), 4, ptr(3), 2, 1, 8, ptr(4), nullptr, ptr(5), ws, 0, -1), MONO_EINVAL);
  EXPECT_CODE(call(ptr(0), ptr(1), 10, nullptr, 4, ptr(3), 2, 1, 8, ptr(4), nullptr, ptr(5), ws, 0, -1), MONO_EINVAL);
  EXPECT_CODE(call(ptr(0), ptr(1), 10, ptr(2), 4, nullptr, 2, 1, 8, ptr(4), nullptr, ptr(5), ws, 0, -1), MONO_EINVAL);
  EXPECT_CODE(call(ptr(0), ptr(1), 10, ptr(2), 4, ptr(3), 2, 1, 8, nullptr, nullptr, ptr(5), ws, 0, -1), MONO_EINVAL);
  EXPECT_CODE(call(ptr(0), ptr(1), 10, ptr(2), 4, ptr(3), 2, 1, 8, ptr(4), nullptr, nullptr, ws, 0, -1), MONO_EINVAL);
  EXPECT_CODE(call(ptr(0), ptr(1), 0, ptr(2), 4, ptr(3), 2, 1, 8, ptr(4), nullptr, ptr(5), ws, 0, -1), MONO_EINVAL);
  EXPECT_CODE(call(misaligned(0), ptr(1), 10, ptr(2), 4, ptr(3), 2, 1, 8, ptr(4), nullptr, ptr(5), ws, 0, -1),
              MONO_EINVAL);
  EXPECT_CODE(call(ptr(0), ptr(1), 10, ptr(2), 4, ptr(3), 2, 1, 8, ptr(4), nullptr,
                   reinterpret_cast<const void*>((uintptr_t)ptr(5) + 128), ws, 0, -1),
              MONO_EINVAL);  // workspace 256-byte alignment
  EXPECT_CODE(call(ptr(0), ptr(1), 10, ptr(2), 4, ptr(3), 2, 1, 600, ptr(4), nullptr, ptr(5), ws, 0, -1),
              MONO_EINVAL);  // k past the table
}

static void check_pa_and_sparse() {
  StepLayout lay{};
  const size_t ws = (size_t)1 << 30;
  const float inf = INFINITY, nan = NAN;
  auto pa = [&](int H, const void* sel, int k, float scale, float ks, float vs, const void* q = ptr(0),
                const void* out = ptr(6), size_t wsb = (size_t)1 << 30) {
    return check_pa_call("pa", q, ptr(1), ptr(2), 10, H, ptr(3), 4, ptr(4), 2, 1, sel, k, scale, ks, vs, out, ptr(7),
                         wsb, &lay);
  };
  EXPECT_CODE(pa(1, nullptr, 0, 0.1f, 1.f, 1.f), MONO_OK);  // dense
  CHECK(lay.sparse == 0 && lay.mode == kModeAttn);
  EXPECT_CODE(pa(1, ptr(5), 16, 0.1f, 1.f, 1.f), MONO_OK);  // sparse
  CHECK(lay.sparse == 1 && lay.k == 16);
  EXPECT_CODE(pa(1, ptr(5), 0, 0.1f, 1.f, 1.f), MONO_EINVAL);
  EXPECT_CODE(pa(0, nullptr, 0, 0.1f, 1.f, 1.f), MONO_ENOTSUP);
  EXPECT_CODE(pa(kMaxHeads + 1, nullptr, 0, 0.1f, 1.f, 1.f), MONO_ENOTSUP);
  EXPECT_CODE(pa(1, nullptr, 0, nan, 1.f, 1.f), MONO_EINVAL);
  EXPECT_CODE(pa(1, nullptr, 0, inf, 1.f, 1.f), MONO_EINVAL);
  EXPECT_CODE(pa(1, nullptr, 0, -inf, 1.f, 1.f), MONO_EINVAL);
  EXPECT_CODE(pa(1, nullptr, 0, 0.1f, 0.f, 1.f), MONO_EINVAL);
  EXPECT_CODE(pa(1, nullptr, 0, 0.1f, -1.f, 1.f), MONO_EINVAL);
  EXPECT_CODE(pa(1, nullptr, 0, 0.1f, 1.f, inf), MONO_EINVAL);
  EXPECT_CODE(pa(1, nullptr, 0, 0.1f, 1.f, nan), MONO_EINVAL);
  EXPECT_CODE(pa(1, nullptr, 0, 0.1f, 1.f, 1.f, nullptr), MONO_EINVAL);
  EXPECT_CODE(pa(1, nullptr, 0, 0.1f, 1.f, 1.f, ptr(0), misaligned(6)), MONO_EINVAL);
  EXPECT_CODE(pa(1, nullptr, 0, 0.1f, 1.f, 1.f, ptr(0), ptr(6), 256), MONO_ENOSPC);

  auto sp = [&](int H, int T, int k, float scale, const void* iq, size_t wsb) {
    return check_sparse_call("sparse", iq, ptr(1), ptr(2), ptr(3), ptr(4), 10, H, ptr(5), 4, ptr(6), 2 * T / T, T, k,
                             scale, 1.f, 1.f, ptr(7), ptr(8), ptr(9), wsb, &lay);
  };
  EXPECT_CODE(sp(1, 1, 64, 0.1f, ptr(0), ws), MONO_OK);
  CHECK(lay.mode == kModeFused && lay.part_splits >= kLocalMaxChunks);  // room for chunk-local splits
  EXPECT_CODE(sp(1, 4, 64, 0.1f, ptr(0), ws), MONO_OK);
  EXPECT_CODE(sp(0, 1, 64, 0.1f, ptr(0), ws), MONO_ENOTSUP);
  EXPECT_CODE(sp(1, 1, 0, 0.1f, ptr(0), ws), MONO_EINVAL);
  EXPECT_CODE(sp(1, 1, 64, nan, ptr(0), ws), MONO_EINVAL);
  EXPECT_CODE(sp(1, 1, 64, 0.1f, nullptr, ws), MONO_EINVAL);
  EXPECT_CODE(sp(1, 1, 64, 0.1f, misaligned(0), ws), MONO_EINVAL);
  EXPECT_CODE(sp(1, 1, 64, 0.1f, ptr(0), 1024), MONO_ENOSPC);
}

static void check_merge_insert_bench() {
  EXPECT_CODE(check_merge_call(ptr(0), ptr(1), 4, 64, 2048, 2048, ptr(2), ptr(3)), MONO_OK);
  EXPECT_CODE(check_merge_call(ptr(0), ptr(1), 4, 64, 2048, 2048, ptr(2), nullptr), MONO_OK);  // scores optional
  EXPECT_CODE(check_merge_call(ptr(0), ptr(1), 5, 64, 2048, 2048, ptr(2), ptr(3)), MONO_ENOTSUP);  // 10240 candidates
  EXPECT_CODE(check_merge_call(ptr(0), ptr(1), 0, 64, 2048, 2048, ptr(2), ptr(3)), MONO_EINVAL);
  EXPECT_CODE(check_merge_call(ptr(0), ptr(1), 4, -1, 2048, 2048, ptr(2), ptr(3)), MONO_EINVAL);
  EXPECT_CODE(check_merge_call(nullptr, nullptr, 4, 0, 2048, 2048, nullptr, nullptr), MONO_OK);  // N = 0: no-op
  EXPECT_CODE(check_merge_call(nullptr, ptr(1), 4, 64, 2048, 2048, ptr(2), ptr(3)), MONO_EINVAL);
  EXPECT_CODE(check_merge_call(misaligned(0), ptr(1), 4, 64, 2048, 2048, ptr(2), ptr(3)), MONO_EINVAL);

  // Indexer context parallelism: shard windows, the candidate budget and
  // the workspace.
  {
    const CpLayout c = cp_layout(64, 1, 4, 256, 2048, 4);
    CHECK(c.shards == 4 && c.width == 64);
    CHECK(c.index.G == 4 && c.index.q_groups == 1);  // the four heads of a token share one scan group
    CHECK(c.cand_idx >= c.index.total && c.cand_scores >= c.cand_idx + (size_t)4 * 256 * 2048 * 4);
    CHECK(c.total == c.cand_scores + (size_t)4 * 256 * 2048 * 4);
    const CpLayout e = cp_layout(2, 1, 3, 5, 100, 8);  // more shards than columns: 5 non-empty windows
    CHECK(e.width == 1 && e.shards == 5);
    const CpLayout m = cp_layout(3, 2, 3, 33, 250, 2);  // (head, token) rows: 6 per request, 2 groups
    CHECK(m.shards == 2 && m.width == 17 && m.index.q_groups == 2);
    CpLayout out;
    const size_t big = (size_t)1 << 40;
    EXPECT_CODE(check_cp_call(ptr(0), ptr(1), 100, ptr(2), 256, ptr(3), 64, 1, 4, 2048, 4, ptr(4), ptr(5), big, &out),
                MONO_OK);
    EXPECT_CODE(check_cp_call(ptr(0), ptr(1), 100, ptr(2), 256, ptr(3), 64, 1, 4, 2048, 5, ptr(4), ptr(5), big, &out),
                MONO_ENOTSUP);  // five shards of 2048 candidates
    EXPECT_CODE(check_cp_call(ptr(0), ptr(1), 100, ptr(2), 256, ptr(3), 64, 1, 0, 2048, 4, ptr(4), ptr(5), big, &out),
                MONO_EINVAL);  // no heads
    EXPECT_CODE(check_cp_call(ptr(0), ptr(1), 100, ptr(2), 256, ptr(3), 64, 1, 4, 2048, 0, ptr(4), ptr(5), big, &out),
                MONO_EINVAL);  // no shards
    EXPECT_CODE(check_cp_call(ptr(0), ptr(1), 100, ptr(2), 256, ptr(3), 64, 1, 4, 2048, 4, nullptr, ptr(5), big, &out),
                MONO_EINVAL);
    EXPECT_CODE(check_cp_call(ptr(0), ptr(1), 100, ptr(2), 256, ptr(3), 64, 1, 4, 2048, 4, ptr(4), ptr(5),
                              cp_layout(64, 1, 4, 256, 2048, 4).total - 1, &out),
                MONO_ENOSPC);
    EXPECT_CODE(check_cp_call(misaligned(0), ptr(1), 100, ptr(2), 256, ptr(3), 64, 1, 4, 2048, 4, ptr(4), ptr(5), big,
                              &out),
                MONO_EINVAL);
  }

  auto ins = [&](const void* kr, const void* vr, const void* ir, int64_t n, int H, const void* kp, const void* vp,
                 const void* ip, int64_t np, const void* err, const void* slots = ptr(9)) {
    return check_insert_call(kr, vr, ir, slots, n, H, kp, vp, ip, np, err);
  };
  EXPECT_CODE(ins(ptr(0), ptr(1), ptr(2), 64, 1, ptr(3), ptr(4), ptr(5), 100, ptr(6)), MONO_OK);
  EXPECT_CODE(ins(nullptr, nullptr, ptr(2), 64, 0, nullptr, nullptr, ptr(5), 100, ptr(6)), MONO_OK);  // index only
  EXPECT_CODE(ins(ptr(0), ptr(1), ptr(2), -1, 1, ptr(3), ptr(4), ptr(5), 100, ptr(6)), MONO_EINVAL);
  EXPECT_CODE(ins(ptr(0), ptr(1), ptr(2), 64, 1, ptr(3), ptr(4), ptr(5), 0, ptr(6)), MONO_EINVAL);
  EXPECT_CODE(ins(ptr(0), ptr(1), ptr(2), 64, 1, nullptr, ptr(4), ptr(5), 100, ptr(6)), MONO_EINVAL);
  EXPECT_CODE(ins(ptr(0), ptr(1), ptr(2), 64, 0, ptr(3), ptr(4), ptr(5), 100, ptr(6)), MONO_ENOTSUP);
  EXPECT_CODE(ins(ptr(0), ptr(1), ptr(2), 64, 1, ptr(3), ptr(4), ptr(5), 100, nullptr), MONO_EINVAL);
  EXPECT_CODE(ins(ptr(0), ptr(1), ptr(2), 64, 1, ptr(3), ptr(4), ptr(5), 100, ptr(6), nullptr), MONO_EINVAL);
  EXPECT_CODE(ins(misaligned(0), ptr(1), ptr(2), 64, 1, ptr(3), ptr(4), ptr(5), 100, ptr(6)), MONO_EINVAL);
  EXPECT_CODE(ins(ptr(0), ptr(1), ptr(2), 64, 1, ptr(3), ptr(4), ptr(5), 100, ptr(6),
                  reinterpret_cast<const void*>((uintptr_t)ptr(9) + 4)),
              MONO_EINVAL);  // slots: 8-byte alignment
  // n x rows per token x 4 < 2^31: 3 rows per token -> n < 178956971
  EXPECT_CODE(ins(ptr(0), ptr(1), ptr(2), 178956970, 1, ptr(3), ptr(4), ptr(5), 100, ptr(6)), MONO_OK);
  EXPECT_CODE(ins(ptr(0), ptr(1), ptr(2), 178956971, 1, ptr(3), ptr(4), ptr(5), 100, ptr(6)), MONO_EINVAL);
  EXPECT_CODE(ins(ptr(0), ptr(1), ptr(2), INT64_MAX / 2, 64, ptr(3), ptr(4), ptr(5), 100, ptr(6)), MONO_EINVAL);

  auto scan = [&](int B, int bts, int cp, int variant, const void* hist = ptr(5)) {
    return check_bench_scan_call(ptr(0), ptr(1), 100, ptr(2), bts, ptr(3), B, cp, variant, hist, ptr(6));
  };
  EXPECT_CODE(scan(64, 256, 32, 0), MONO_OK);
  EXPECT_CODE(scan(64, 256, 32, 1), MONO_OK);
  EXPECT_CODE(scan(64, 256, 33, 0), MONO_EINVAL);  // 33 pages exceed the LDS score area
  EXPECT_CODE(scan(64, 256, 0, 0), MONO_EINVAL);
  EXPECT_CODE(scan(64, 256, 32, 2), MONO_EINVAL);
  EXPECT_CODE(scan(0, 256, 32, 0), MONO_EINVAL);
  EXPECT_CODE(scan(64, 256, 32, 0, nullptr), MONO_EINVAL);
  EXPECT_CODE(check_bench_read_call(ptr(0), nullptr, 16, 0, 512, ptr(1)), MONO_OK);
  EXPECT_CODE(check_bench_read_call(ptr(0), ptr(2), 16, 1, 512, ptr(1)), MONO_OK);
  EXPECT_CODE(check_bench_read_call(ptr(0), nullptr, 16, 1, 512, ptr(1)), MONO_EINVAL);  // gather needs ids
  EXPECT_CODE(check_bench_read_call(ptr(0), nullptr, 16, 2, 512, ptr(1)), MONO_EINVAL);
  EXPECT_CODE(check_bench_read_call(ptr(0), nullptr, 0, 0, 512, ptr(1)), MONO_EINVAL);
  EXPECT_CODE(check_bench_read_call(ptr(0), nullptr, 16, 0, 0, ptr(1)), MONO_EINVAL);
  EXPECT_CODE(check_bench_read_call(ptr(0), nullptr, 16, 0, 65537, ptr(1)), MONO_EINVAL);
  EXPECT_CODE(check_bench_read_call(misaligned(0), nullptr, 16, 0, 512, ptr(1)), MONO_EINVAL);
}

// Layout invariants: regions 256-byte aligned, in order, inside the total.
static void check_layout(const StepLayout& l) {
  const size_t regions[] = {l.err,  l.ctrl_base, l.hist,   l.hist2, l.hist3, l.ties, l.xcand,
                            l.xcnt, l.scores,    l.cand,   l.pm,    l.pl,    l.pacc};
  size_t prev = 0;
  for (size_t r : regions) {
    CHECK(r % 256 == 0);
    CHECK(r >= prev);
    prev = r;
  }
  CHECK(l.total >= prev);
  CHECK(l.ctrl_base == 256 && l.zero_end >= l.ctrl_base + l.ctrl_words * 4 && l.zero_end <= l.scores);
  CHECK(l.xcnt <= l.zero_end);  // the exchanged pairs and counts start at zero (a written entry is never 0)
  CHECK(l.zero_units == (l.zero_end >> 8));
  CHECK((size_t)l.n_clear * kClearBytes + l.ctrl_base + kHdrWords * 4 >= l.zero_end);
  CHECK(l.queue + l.n_queue <= l.ctrl_words);
}

// Plan invariants for a call of the given shape on a device.
static void check_plan(int mode, int B, int T, int H, int bts, int k, bool fp8, bool sel_scores, int lo, int hi,
                       const DeviceShape& dev, int G = 1) {
  const int sparse = (mode & kModeIndex) ? 1 : (k > 0);
  const StepLayout l0 = step_layout(mode, B, T, H, bts, k, sparse, G);
  check_layout(l0);
  StepLayout l = l0;
  if (lo >= 0) {
    l.win_lo = lo;
    l.win_hi = hi;
  }
  int variant = -1;
  const long grid = plan_step(l, dev, fp8, sel_scores, &variant, "plan");
  CHECK(grid > 0);
  CHECK(variant >= 0 && variant < kStepVariants);
  CHECK(grid <= dev.resident[variant]);
  if (mode & kModeAttn) {
    const long list_max = sparse ? k : (long)bts * kPageTokens;
    CHECK((long)l.n_splits * l.split_tokens >= list_max);
    CHECK(l.n_splits <= l0.part_splits);  // the partial buffers hold every split
  }
  if (mode & kModeIndex) CHECK((long)l.chunks * l.chunk_pages >= l.win_hi - l.win_lo);
  if (l.local) {
    CHECK(mode == kModeFused && T == 1 && !sel_scores && l.win_lo == 0);
    CHECK(variant == local_variant(fp8));
    CHECK(l.chunk_pages * kPageTokens <= kLocalTokens && l.chunks <= kLocalMaxChunks);
    // every chunk item is a first-round item of a grid that fits at once
    CHECK((long)B * l.chunks == (long)l.n_scan && (long)l.n_scan <= grid && grid <= dev.resident[variant]);
    CHECK(l.n_queue == 0u);
  } else if (mode == kModeAttn && dev.resident[attn_variant(fp8)] > 0) {
    CHECK(variant == attn_variant(fp8));  // the attention call's own instance
  } else {
    CHECK(variant == step_variant(G * T > 1 && (mode & kModeIndex), fp8));
  }
  if (l.local_filter) {
    // scan chunks filter their own scores: one row per request, chunks of
    // one slice, every chunk a first-round item (they wait for the row's
    // histogram), and no filter items in the queue
    CHECK(!l.local && (mode & kModeIndex) && G == 1 && T == 1 && !l.select_mode && !sel_scores && l.win_lo == 0);
    CHECK(l.chunk_pages * kPageTokens <= kSlice && (long)l.n_scan <= grid && l.n_filter == 0u);
    CHECK(l.n_queue == l.n_select + l.n_attn);
  }
}

static void check_plans() {
  DeviceShape mi{};
  mi.cus = 256;
  for (int v = 0; v < kStepVariants; ++v) mi.resident[v] = 512;  // two 4-wave workgroups per compute unit

  // The one-launch step of batch 64 x 32768 tokens, top 2048: chunk-local,
  // 8 chunks of 32 pages per request, 512 workgroups.
  {
    StepLayout l = step_layout(kModeFused, 64, 1, 1, 256, 2048, 1);
    int variant = -1;
    const long grid = plan_step(l, mi, false, false, &variant, "w3");
    CHECK(l.local == 1 && variant == local_variant(false) && grid == 512);
    CHECK(l.chunks == 8 && l.chunk_pages == 32 && l.n_scan == 512u);
  }
  // One resident workgroup short: the chunk-local instance is refused and
  // the item-queue instance runs instead.
  {
    DeviceShape d = mi;
    d.resident[local_variant(false)] = 511;
    StepLayout l = step_layout(kModeFused, 64, 1, 1, 256, 2048, 1);
    int variant = -1;
    const long grid = plan_step(l, d, false, false, &variant, "w3-short");
    CHECK(l.local == 0 && variant == step_variant(false, false) && grid > 0 && grid <= 512);
    d.resident[local_variant(false)] = 0;  // no occupancy figure at all
    l = step_layout(kModeFused, 64, 1, 1, 256, 2048, 1);
    plan_step(l, d, false, false, &variant, "w3-none");
    CHECK(l.local == 0);
  }
  // The same with fp8 pages, with selected scores requested, or with four
  // query tokens per request: never chunk-local with scores or T > 1.
  {
    StepLayout l = step_layout(kModeFused, 64, 1, 1, 256, 2048, 1);
    int variant = -1;
    plan_step(l, mi, true, false, &variant, "fp8");
    CHECK(l.local == 1 && variant == local_variant(true));
    l = step_layout(kModeFused, 64, 1, 1, 256, 2048, 1);
    plan_step(l, mi, false, true, &variant, "scores");
    CHECK(l.local == 0);
    l = step_layout(kModeFused, 128, 4, 1, 512, 2048, 1);
    plan_step(l, mi, false, false, &variant, "t4");
    CHECK(l.local == 0 && variant == step_variant(true, false));
    // 512 query tokens: two splits of 1024 each (two rounds of workgroups),
    // within the 8 splits the partial buffers hold.
    CHECK(l.split_tokens == 1024 && l.n_splits == 2 && l.n_attn == 1024u && l.n_splits <= l.part_splits);
    // The attention call alone keeps one round: one split per query token.
    l = step_layout(kModeAttn, 128, 4, 1, 512, 2048, 1);
    plan_step(l, mi, false, false, &variant, "t4-attn");
    CHECK(l.n_splits == 1 && l.n_attn == 512u);
  }
  // Long rows (8 x 262144 tokens): a chunk would exceed the LDS score area;
  // the item-queue instance runs, its 512 scan chunks filtering their own
  // scores.  With one resident workgroup short, the chunks publish filter
  // items instead.
  {
    StepLayout l = step_layout(kModeFused, 8, 1, 1, 2048, 4096, 1);
    int variant = -1;
    plan_step(l, mi, false, false, &variant, "long");
    CHECK(l.local == 0 && l.split_tokens == 256 && l.n_splits == 16);
    CHECK(l.local_filter == 1 && l.n_scan == 512u && l.n_filter == 0u);
    DeviceShape d = mi;
    d.resident[step_variant(false, false)] = 511;
    l = step_layout(kModeFused, 8, 1, 1, 2048, 4096, 1);
    plan_step(l, d, false, false, &variant, "long-short");
    CHECK(l.local_filter == 0 && l.n_filter > 0u);
  }
  // Dense attention, batch 32 x 8192 tokens: the attention-only instance,
  // one split of 512 tokens per resident workgroup.
  {
    StepLayout l = step_layout(kModeAttn, 32, 1, 1, 64, 0, 0);
    int variant = -1;
    const long grid = plan_step(l, mi, false, false, &variant, "w2");
    CHECK(variant == attn_variant(false) && grid == 512 && l.split_tokens == 512 && l.n_splits == 16);
  }
  // Workload shapes and random shapes: plan invariants.
  check_plan(kModeAttn, 1, 1, 1, 2, 0, false, false, -1, -1, mi);
  check_plan(kModeAttn, 32, 1, 1, 64, 0, false, false, -1, -1, mi);
  check_plan(kModeFused, 64, 1, 1, 256, 2048, false, false, -1, -1, mi);
  check_plan(kModeFused, 128, 4, 1, 512, 2048, false, false, -1, -1, mi);
  check_plan(kModeFused, 8, 1, 1, 2048, 4096, false, false, -1, -1, mi);
  check_plan(kModeIndex, 256, 1, 1, 64, 2048, false, false, 16, 32, mi);  // one shard's page window
  std::mt19937 rng(7);
  for (int it = 0; it < 3000; ++it) {
    const int mode = 1 + (int)(rng() % 3);
    const int B = 1 + (int)(rng() % 300), T = 1 + (int)(rng() % 8), H = 1 + (int)(rng() % 3);
    const int bts = 1 + (int)(rng() % 2100);
    const int kmax = bts * kPageTokens;
    const int k = (mode == kModeAttn && rng() % 2) ? 0 : 1 + (int)(rng() % std::min(kmax, 9000));
    DeviceShape d{};
    d.cus = 8 * (1 + (int)(rng() % 40));
    for (int v = 0; v < kStepVariants; ++v) d.resident[v] = d.cus * (1 + (int)(rng() % 3)) - (int)(rng() % 3);
    const bool fp8 = rng() % 2, scores = (mode & kModeIndex) && rng() % 4 == 0;
    int lo = -1, hi = -1;
    if (mode == kModeIndex && rng() % 3 == 0) {
      lo = (int)(rng() % bts);
      hi = lo + 1 + (int)(rng() % (bts - lo));
    }
    const int G = mode == kModeIndex ? 1 + (int)(rng() % 5) : 1;  // index heads (context parallelism)
    check_plan(mode, B, T, H, bts, k, fp8, scores, lo, hi, d, G);
  }
}

int main() {
  check_shapes();
  check_pages();
  check_index();
  check_pa_and_sparse();
  check_merge_insert_bench();
  check_plans();
  printf("host_check: %d checks, %d failed\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
