// One persistent work-queue kernel runs every step of the path (gfx950).
//
// Work items:
//   scan   (request b, query group, chunk of 16 index pages)  -> scan_chunk
//   select (query token i), for score rows of at most 64K      -> select_query
//   filter (query token i, slice of 4096 scores), longer rows  -> filter_slice,
//          and the last slice of i to finish                   -> resolve_query
//   attn   (query token i, KV head h, split of candidates)    -> attn_split
//          (the last split of (i, h) to finish merges them)
// mono_index_score_topk runs the scan and filter items, mono_pa_decode_mxfp4
// the attention items, mono_sparse_decode_mxfp4 all three in one launch.
// With one query token per request, mono_sparse_decode_mxfp4 runs a separate
// instance whose only items are chunk-local steps (local_item): each chunk
// scans, selects together with the other chunks of its request, and attends
// over its own share of the selection.
//
// Workgroups take tickets from one atomic counter.  The first tickets are
// the items that are ready at the start (the scans, or the attention splits
// of the attention call); every later ticket is a slot of a ready queue.
// An item that completes a dependency publishes the items it unblocks: the
// last scan chunk of a query group publishes the group's select items or
// filter slices (or, with one query token per request and a short row,
// selects it at once), and whoever completes a query token's selection
// publishes the token's attention splits.  So no item ever waits
// for another; a workgroup only waits for its queue slot to be filled, and
// the number of published items is fixed by the shapes, so every slot is
// filled (every wait is also bounded and flags MONO_DEVERR_WAIT).  The last
// workgroup to leave resets the queue and all counters for the next call.
#include "attn_device.h"
#include "mono_decode.h"
#include "topk_device.h"

#include <mutex>

namespace mono {

constexpr uint32_t kMaxSpins = 1u << 21;  // bound of one wait (seconds, far above any step)
constexpr int kPairReadDelay = 32;  // s_sleep units (64 cycles each) before the first read of exchanged pairs: ~0.85 us

namespace {

// A clear item: zero bytes [c * kClearBytes, ...) of the region that must
// start at zero.  Coherent stores, so atomics of other workgroups that run
// on other dies see the zeros rather than stale data.
__device__ __forceinline__ void clear_item(const StepLayout& lay, uint32_t c, uint8_t* ws, uint32_t* ctrl) {
  const size_t begin = lay.ctrl_base + kHdrWords * 4 + (size_t)c * kClearBytes;
  const size_t end = min(begin + (size_t)kClearBytes, lay.zero_end);
  uint32_t* p = reinterpret_cast<uint32_t*>(ws + begin);
  const int n = (int)((end - begin) / 4);
  for (int x = thread_index(); x < n; x += kBlock) store_coherent(p + x, 0u);
  wait_vmem();
  __syncthreads();
  if (thread_index() == 0) atomicAdd(ctrl + kHdrCleared, 1u);
}

// A bounded wait that ran out: the error bit, and the workspace's zero
// record dropped so that the next call clears the control block before it
// starts (a late producer may still fill a slot or count an arrival after
// the counters' last users have reset them).
__device__ __forceinline__ void wait_ran_out(uint32_t* err, uint32_t* ctrl) {
  raise_error(err, kErrWait);
  store_coherent(ctrl + kHdrZeroed, 0u);
}

// Thread 0 waits until *p >= target; everyone leaves together.
__device__ __forceinline__ void wait_counter(const uint32_t* p, uint32_t target, uint32_t* err, uint32_t* ctrl) {
  if (thread_index() == 0) {
    uint32_t spins = 0;
    while (load_coherent(p) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kMaxSpins) {
        wait_ran_out(err, ctrl);
        break;
      }
    }
  }
  __syncthreads();
}

// Thread 0 waits until queue slot q is filled; returns its descriptor to
// every thread (0 if the bounded wait ran out: the slot is then skipped).
__device__ __forceinline__ uint32_t wait_slot(const uint32_t* q, uint32_t* err, uint32_t* ctrl, uint32_t& s_desc) {
  if (thread_index() == 0) {
    uint32_t spins = 0, d;
    while ((d = load_coherent(q)) == 0u) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kMaxSpins) {
        wait_ran_out(err, ctrl);
        break;
      }
    }
    s_desc = d;
    if (d) *const_cast<uint32_t*>(q) = 0u;  // the slot's one consumer leaves it empty for the next call
  }
  __syncthreads();
  const uint32_t d = s_desc;
  __syncthreads();
  return d;
}

// Publish items first..first+count-1 of one kind into the ready queue.
// Called by every thread of the workgroup after its own results are
// complete (wait_vmem and a barrier), so consumers see them.
__device__ __forceinline__ void publish(const StepLayout& lay, uint32_t* ctrl, uint32_t kind, uint32_t first,
                                        uint32_t count, uint32_t* err, uint32_t& s_base) {
  if (thread_index() == 0) {
    s_base = atomicAdd(ctrl + lay.pub, count);
    // The publications add up to the queue's length: the last one leaves
    // the counter at zero for the next call.
    if (s_base + count == lay.n_queue) ctrl[lay.pub] = 0u;
  }
  __syncthreads();
  const uint32_t base = s_base;
  if (base + count > lay.n_queue) {  // never expected: the counts are fixed by the shapes
    if (thread_index() == 0) raise_error(err, kErrSelection);
    return;
  }
  for (uint32_t x = thread_index(); x < count; x += kBlock)
    store_coherent(ctrl + lay.queue + base + x, (kind << kKindShift) | (first + x));
}

// Index row of request b's (head, token) pair u = h * T + t.
__device__ __forceinline__ int index_row(const StepLayout& lay, int b, int u) {
  return (u / lay.T) * (lay.B * lay.T) + b * lay.T + u % lay.T;
}

// Request and query token of index row i.
__device__ __forceinline__ void row_request(const StepLayout& lay, int i, int& b, int& t) {
  const int r = i % (lay.B * lay.T);
  b = r / lay.T;
  t = r % lay.T;
}

// Tokens query position pos sees inside the layout's page window (all of
// 0..pos unless the index call was given a window).
__device__ __forceinline__ int window_valid(const StepLayout& lay, int pos) {
  return max(0, min(pos + 1, lay.win_hi * kPageTokens) - lay.win_lo * kPageTokens);
}

// ---------------------------------------------------------------------------
// Chunk-local step (the one-launch call with one query token per request).
// The scan item of chunk c keeps its scores in LDS.  The chunks of a request
// are all resident at once, so they can agree on the threshold of the k-th
// largest score through global histograms, one radix level at a time (key
// bits 31..21, 20..10, 9..0; a level runs only while the threshold bin
// holds more tokens than places left): each chunk adds its counts, arrives,
// waits for the others and reads the sums.  More exact ties at the final key
// than places go to the lowest positions, chunk by chunk, through per-chunk
// tie counts.  Every chunk then attends over its own selected tokens as one
// split of the token's attention; the last split to arrive merges them.
// Scores, candidates and the selection never travel through global memory
// between items, and no item is queued.
// ---------------------------------------------------------------------------
struct LocalLds {
  union {
    struct {
      float scores[kLocalTokens];  // token e of the chunk (position 128 * first page + e)
      ScanLds<1> scan;             // the scan's histogram, then each level's
    } sel;
    AttnLds attn;  // the attention's combine area (its block-table part is unused)
  } u;
  uint16_t list[kLocalTokens];  // the chunk's selected tokens e
  int32_t ptab[kLocalTokens / kPageTokens];
  uint32_t scratch[kWaves + 4];
  uint32_t xc[kLocalMaxChunks], xpre[kLocalMaxChunks + 1];  // exchanged counts per chunk, their prefix sums
};
static_assert(sizeof(float) * kLocalTokens >= sizeof(uint2) * kExchCap, "exchanged candidates reuse the score area");

// A one-row scan item's scores, staged in LDS and written out whole at the
// end of the chunk (a scan loop with no global stores keeps its page loads
// in flight), with the chunk's page ids.
struct ScanStageLds {
  ScanLds<1> scan;
  float scores[kMaxChunkPages * kPageTokens];
  int32_t ptab[kMaxChunkPages];
};

template <int TQ>
union StepLds {
  ScanLds<TQ> scan;
  ScanStageLds stage;  // TQ 1
  FilterLds filter;
  ResolveLds resolve;
  AttnLds attn;
};

// Selection arguments of query token i.
__device__ __forceinline__ SelectArgs select_args(const StepArgs& a, const StepLayout& lay, int i, int n_valid,
                                                  uint32_t* ctrl, uint32_t* err) {
  SelectArgs sa;
  sa.scores = reinterpret_cast<const float*>(a.ws + lay.scores) + (size_t)i * lay.lcap;
  sa.lcap = lay.lcap;
  sa.ghist = reinterpret_cast<uint32_t*>(a.ws + lay.hist) + (size_t)i * kHistBins;
  sa.out = a.sel + (size_t)i * lay.k;
  sa.out_scores = a.sel_scores ? a.sel_scores + (size_t)i * lay.k : nullptr;
  sa.out_cnt = ctrl + lay.out_cnt + i;
  sa.cand = reinterpret_cast<uint64_t*>(a.ws + lay.cand) + (size_t)i * kCandCap;
  sa.cand_cnt = ctrl + lay.cand_cnt + i;
  sa.err = err;
  sa.n_valid = n_valid;
  sa.j_base = lay.win_lo * kPageTokens;
  sa.k = lay.k;
  return sa;
}

// Whole selection of query token i (if its request is valid), then, in the
// one-launch step, publication of its attention splits.
template <int TQ>
__device__ __forceinline__ void select_item(const StepArgs& a, const StepLayout& lay, uint32_t i, StepLds<TQ>& lds,
                                            uint32_t* ctrl, uint32_t* err, uint32_t& s_pub) {
  const int T = lay.T;
  int b, t;
  row_request(lay, (int)i, b, t);
  const int L = a.seq_lens[b];
  if (L >= T && L <= lay.lcap) {  // an invalid length was reported by the scan items
    select_query(select_args(a, lay, (int)i, window_valid(lay, L - T + t), ctrl, err), lds.resolve);
    wait_vmem();
    MONO_STAMP(17);
  }
  __syncthreads();
  if (lay.mode == kModeFused)
    publish(lay, ctrl, kItemAttn, i * (uint32_t)(lay.H * lay.n_splits), (uint32_t)(lay.H * lay.n_splits), err, s_pub);
}

// Every thread's memory updates are complete, then this workgroup arrives at
// *cnt and waits until `target` workgroups have.  The arrival returns the
// count, so the last workgroup to arrive does not poll.
__device__ __forceinline__ void arrive_wait(uint32_t* cnt, uint32_t target, uint32_t* err, uint32_t* ctrl) {
  wait_vmem();
  __syncthreads();
  if (thread_index() == 0 && atomicAdd(cnt, 1u) + 1u < target) {
    uint32_t spins = 0;
    while (load_coherent(cnt) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kMaxSpins) {
        wait_ran_out(err, ctrl);
        break;
      }
    }
  }
  __syncthreads();
}

// Adds the digits (key >> shift) & (nbins - 1) of this thread's keys marked
// in `mask` to global histogram row g, through an LDS histogram.
__device__ __forceinline__ void level_counts(const uint32_t* key, uint32_t mask, int shift, int nbins, uint32_t* hist,
                                             uint32_t* g) {
  const int tid = thread_index();
  for (int x = tid; x < nbins; x += kBlock) hist[x] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 16; ++u)
    if ((mask >> u) & 1u) atomicAdd(&hist[(key[u] >> shift) & (uint32_t)(nbins - 1)], 1u);
  __syncthreads();
  for (int x = tid; x < nbins; x += kBlock) {
    const uint32_t v = hist[x];
    if (v) atomicAdd(g + x, v);
  }
}

template <class Fmt>
__device__ __forceinline__ void local_item(const StepArgs& a, const StepLayout& lay, uint32_t t, LocalLds& lds,
                                           uint32_t* ctrl, uint32_t* err) {
  const int tid = thread_index();
  // Workgroups are dealt to the 8 XCDs in turn (workgroup x to XCD x % 8),
  // and the first ticket of each is its index.  XCD x takes one contiguous
  // run of the (request, chunk) pairs in request-major order, so the chunks
  // of a request, which hand data to each other, mostly share an XCD.
  uint32_t pair;
  {
    const uint32_t n = lay.n_scan, q = n >> 3, r = n & 7u, x = t & 7u, y = t >> 3;
    pair = x * q + min(x, r) + y;
  }
  const int b = (int)(pair / (uint32_t)lay.chunks), c = (int)(pair % (uint32_t)lay.chunks);
  const int L = a.seq_lens[b];
  if (L < 1 || L > lay.lcap) {
    if (c == 0 && tid == 0) raise_error(err, kErrSeqLen);
    return;
  }
  const int n_pages = (L + kPageTokens - 1) / kPageTokens;
  const int nch = (n_pages + lay.chunk_pages - 1) / lay.chunk_pages;
  if (c >= nch) return;  // every chunk of the request agrees on nch
  const int i = b;       // one query token per request, at position L - 1; tokens 0..L-1 are valid
  const int p_begin = c * lay.chunk_pages, p_end = min(p_begin + lay.chunk_pages, n_pages);
  const int tok0 = p_begin * kPageTokens;
  const int n_mine = min(L, p_end * kPageTokens) - tok0;  // valid tokens of the chunk (>= 1)
  const int k = lay.k;
  uint32_t* g1 = reinterpret_cast<uint32_t*>(a.ws + lay.hist) + (size_t)i * kHistBins;
  uint32_t* g2 = reinterpret_cast<uint32_t*>(a.ws + lay.hist2) + (size_t)i * kHistBins;
  uint32_t* g3 = reinterpret_cast<uint32_t*>(a.ws + lay.hist3) + (size_t)i * 1024;
  uint32_t* gt = reinterpret_cast<uint32_t*>(a.ws + lay.ties) + (size_t)i * kLocalMaxChunks;
  uint32_t* lvl = ctrl + lay.lvl_cnt + (size_t)i * kLvlWords;
  uint32_t* hist = lds.u.sel.scan.hist;

  {
    ScanArgs sa;
    sa.index_q = a.index_q;
    sa.pages = a.index_pages;
    sa.num_pages = a.num_pages;
    sa.bt_row = a.block_table + (size_t)b * a.bt_stride;
    sa.scores = nullptr;
    sa.ghist = reinterpret_cast<uint32_t*>(a.ws + lay.hist);  // row i: g1
    sa.err = err;
    sa.lcap = lay.lcap;
    sa.row[0] = sa.row[1] = sa.row[2] = sa.row[3] = i;
    sa.pos[0] = sa.pos[1] = sa.pos[2] = sa.pos[3] = L - 1;
    sa.tq = 1;
    sa.p_begin = p_begin;
    sa.p_end = p_end;
    scan_chunk<1, Fmt, true>(sa, lds.u.sel.scan, (lds_f32*)lds.u.sel.scores, (lds_i32w*)lds.ptab);
  }
  __syncthreads();
  MONO_STAMP(2);

  // Thread t holds the keys of tokens 16t..16t+15 of the chunk.
  uint32_t key[16];
  {
    const f32x4_t* sp = reinterpret_cast<const f32x4_t*>(lds.u.sel.scores + 16 * tid);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4_t v = sp[q4];
#pragma unroll
      for (int x = 0; x < 4; ++x) key[4 * q4 + x] = score_key(v[x]);
    }
  }
  const int n_here = max(0, min(16, n_mine - 16 * tid));
  const uint32_t valid = n_here >= 16 ? 0xFFFFu : ((1u << n_here) - 1u);

  // Threshold: every token with key > thr is selected, and of those with
  // key == thr the first `take` in position order (all of them unless ties).
  const bool all = L <= k;
  uint32_t thr = 0u, take = 0xFFFFFFFFu;
  bool ties = false, exchanged = false;
  if (!all) {
    // The request's histogram row is complete once it counts all L tokens
    // (counts only grow): every chunk reads the row until it does, so the
    // row's last update is seen one round trip after it lands, with no
    // arrival counter in between.
    BinSplit s1;
    for (uint32_t spins = 0;; ++spins) {
      uint32_t total;
      s1 = find_bin_of_rank_global<kHistBins>(g1, (uint32_t)k, lds.scratch, &total);
      if (total == (uint32_t)L) break;  // the same in every thread
      if (spins > kMaxSpins) {
        if (tid == 0) wait_ran_out(err, ctrl);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    MONO_STAMP(3);
    MONO_STAMP(4);
    uint32_t R = (uint32_t)k - s1.above;
    const uint32_t B1 = (uint32_t)s1.bin;
    thr = B1 << kHistShift;
    if (s1.count != R && s1.count <= (uint32_t)kExchCap) {
      // Few enough tokens in bin B1: every chunk publishes its own (key,
      // position) pairs of that bin, then each chunk reads all of them and
      // takes the rest of the selection from them in LDS.
      uint32_t m2 = 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) m2 |= ((key[u] >> kHistShift) == B1) ? (1u << u) : 0u;
      m2 &= valid;
      uint32_t my_cnt;
      const uint32_t my_off = block_exclusive_scan((uint32_t)__popc(m2), lds.scratch, my_cnt);
      uint64_t* xc_all = reinterpret_cast<uint64_t*>(a.ws + lay.xcand) + (size_t)i * kLocalMaxChunks * kExchCap;
      uint32_t* xn_all = reinterpret_cast<uint32_t*>(a.ws + lay.xcnt) + (size_t)i * kLocalMaxChunks;
      // A written entry is never zero (the position is stored plus one) and
      // a written count is the count plus one: every chunk reads the pairs
      // until each chunk's count and entries are in, so the last chunk's
      // pairs are seen one round trip after they land, with no arrival
      // counter and no wait for the stores' completion.  The last chunk to
      // finish its reads zeroes them again.
      {
        uint64_t* mine = xc_all + (size_t)c * kExchCap;
        uint32_t bits = m2, o = my_off;
        while (bits) {
          const int u = __builtin_ctz(bits);
          bits &= bits - 1u;
          store_coherent(mine + o++, (uint64_t)key[u] | ((uint64_t)(uint32_t)(tok0 + 16 * tid + u + 1) << 32));
        }
      }
      if (tid == 0) store_coherent(xn_all + c, my_cnt + 1u);
      MONO_STAMP(5);
      exchanged = true;
      // Counts and the first `win` entries of every chunk are requested at
      // once (win: a power of two, nch * win <= kExchCap); chunks with more
      // follow in a second round.
      const int win_log2 = 11 - (32 - __builtin_clz((uint32_t)(nch - 1) | 1u)) + (nch == 1 ? 1 : 0);
      const int win = 1 << win_log2;
      constexpr int kPer = kExchCap / kBlock;
      uint64_t v[kPer];
      // Every chunk of the request stores its pairs at about the same time
      // (they all see the histogram complete together), so a read issued at
      // once mostly finds some missing and costs a second round trip; the
      // first read waits about as long as the stores take to land.
      __builtin_amdgcn_s_sleep(kPairReadDelay);
      for (uint32_t spins = 0;; ++spins) {
        const uint32_t cnt_ld = tid < nch ? load_coherent(xn_all + tid) : 0u;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int e = q * kBlock + tid, cc = e >> win_log2, r = e & (win - 1);
          v[q] = cc < nch ? load_coherent(xc_all + (size_t)cc * kExchCap + r) : 0ull;
        }
        if (tid < nch) lds.xc[tid] = cnt_ld;
        __syncthreads();
        bool missing = false;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int e = q * kBlock + tid, cc = e >> win_log2, r = e & (win - 1);
          if (cc < nch) {
            const uint32_t c1 = lds.xc[cc];  // count + 1, or 0 while unwritten
            missing |= c1 == 0u || ((uint32_t)r + 1u < c1 && v[q] == 0ull);
          }
        }
        if (!__syncthreads_or(missing)) break;
        if (spins > kMaxSpins) {
          if (tid == 0) wait_ran_out(err, ctrl);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (tid < nch) lds.xc[tid] = max(lds.xc[tid], 1u) - 1u;
      __syncthreads();
      if (tid == 0) {
        uint32_t acc = 0;
        for (int cc = 0; cc < nch; ++cc) {
          lds.xpre[cc] = acc;
          acc += min(lds.xc[cc], (uint32_t)kExchCap);
        }
        lds.xpre[nch] = acc;
      }
      __syncthreads();
      uint2* cand = reinterpret_cast<uint2*>(lds.u.sel.scores);
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int e = q * kBlock + tid, cc = e >> win_log2, r = e & (win - 1);
        if (cc < nch && (uint32_t)r < lds.xc[cc]) {
          const uint32_t at = lds.xpre[cc] + (uint32_t)r;
          if (at < (uint32_t)kExchCap) cand[at] = make_uint2((uint32_t)v[q], (uint32_t)(v[q] >> 32) - 1u);
        }
      }
      for (int cc = 0; cc < nch; ++cc) {
        const uint32_t n_cc = min(lds.xc[cc], (uint32_t)kExchCap);
        for (uint32_t r = (uint32_t)win + tid; r < n_cc; r += kBlock) {
          const uint32_t at = lds.xpre[cc] + r;
          uint64_t x;
          uint32_t spins = 0;
          while ((x = load_coherent(xc_all + (size_t)cc * kExchCap + r)) == 0ull) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kMaxSpins) {
              wait_ran_out(err, ctrl);
              break;
            }
          }
          if (at < (uint32_t)kExchCap) cand[at] = make_uint2((uint32_t)x, (uint32_t)(x >> 32) - 1u);
        }
      }
      MONO_STAMP(7);
      const int n_c = (int)min(lds.xpre[nch], (uint32_t)kExchCap);
      if (lds.xpre[nch] != s1.count && tid == 0) raise_error(err, kErrSelection);  // never expected
      // A radix pass over key bits 20..10 among the candidates (each
      // thread's share held in registers), then the rest within the
      // threshold sub-bin.
      for (int x = tid; x < kHistBins; x += kBlock) hist[x] = 0u;
      if (tid == 0) lds.scratch[kWaves + 3] = 0u;  // survivor count
      __syncthreads();  // and every candidate is in LDS
      uint32_t ck[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) ck[q] = q * kBlock + tid < n_c ? cand[q * kBlock + tid].x : 0u;
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        if (q * kBlock + tid < n_c) atomicAdd(&hist[(ck[q] >> 10) & 0x7FFu], 1u);
      __syncthreads();
      const BinSplit s2 = find_bin_of_rank(hist, kHistBins, R, lds.scratch);
      R -= s2.above;
      const uint32_t pre2 = (B1 << 11) | (uint32_t)s2.bin;
      thr = pre2 << 10;
      if (s2.count != R && s2.count <= (uint32_t)kBlock) {
        // The sub-bin's keys (a few, as a rule) are compacted into the free
        // histogram words; the one whose count of larger keys is below R
        // and reaches R with its equals is the R-th largest.
        uint32_t* skey = hist;
#pragma unroll
        for (int q = 0; q < kPer; ++q)
          if (q * kBlock + tid < n_c && (ck[q] >> 10) == pre2) skey[atomicAdd(&lds.scratch[kWaves + 3], 1u)] = ck[q];
        __syncthreads();
        const uint32_t n_surv = s2.count;
        if (tid < (int)n_surv) {
          const uint32_t mk = skey[tid];
          uint32_t gt = 0, eq = 0;
          for (uint32_t o = 0; o < n_surv; ++o) {
            const uint32_t ok = skey[o];
            gt += ok > mk ? 1u : 0u;
            eq += ok == mk ? 1u : 0u;
          }
          if (gt < R && R <= gt + eq) {  // every such thread holds the same key: same values
            lds.scratch[kWaves] = mk;
            lds.scratch[kWaves + 1] = gt;
            lds.scratch[kWaves + 2] = eq;
          }
        }
        __syncthreads();
        thr = lds.scratch[kWaves];
        R -= lds.scratch[kWaves + 1];
        if (lds.scratch[kWaves + 2] != R) {
          // More tokens with key thr than places: the lowest positions
          // first; `before` counts those of the chunks ahead of this one.
          uint32_t mine = 0;
          for (int e = tid; e < n_c; e += kBlock) mine += (cand[e].x == thr && (int)cand[e].y < tok0) ? 1u : 0u;
          uint32_t before;
          block_exclusive_scan(mine, lds.scratch, before);
          take = R > before ? R - before : 0u;
          ties = true;
        }
      } else if (s2.count != R) {
        for (int x = tid; x < 1024; x += kBlock) hist[x] = 0u;
        __syncthreads();
        for (int e = tid; e < n_c; e += kBlock)
          if ((cand[e].x >> 10) == pre2) atomicAdd(&hist[cand[e].x & 0x3FFu], 1u);
        __syncthreads();
        const BinSplit s3 = find_bin_of_rank(hist, 1024, R, lds.scratch);
        R -= s3.above;
        thr = (pre2 << 10) | (uint32_t)s3.bin;
        if (s3.count != R) {
          // More tokens with key thr than places: the lowest positions
          // first; `before` counts those of the chunks ahead of this one.
          uint32_t mine = 0;
          for (int e = tid; e < n_c; e += kBlock) mine += (cand[e].x == thr && (int)cand[e].y < tok0) ? 1u : 0u;
          uint32_t before;
          block_exclusive_scan(mine, lds.scratch, before);
          take = R > before ? R - before : 0u;
          ties = true;
        }
      }
    } else if (s1.count != R) {
      uint32_t m2 = 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) m2 |= ((key[u] >> kHistShift) == B1) ? (1u << u) : 0u;
      level_counts(key, m2 & valid, 10, kHistBins, hist, g2);
      arrive_wait(lvl + 1, (uint32_t)nch, err, ctrl);
      const BinSplit s2 = find_bin_of_rank_global<kHistBins>(g2, R, lds.scratch);
      R -= s2.above;
      const uint32_t pre2 = (B1 << 11) | (uint32_t)s2.bin;
      thr = pre2 << 10;
      if (s2.count != R) {
        uint32_t m3 = 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) m3 |= ((key[u] >> 10) == pre2) ? (1u << u) : 0u;
        level_counts(key, m3 & valid, 0, 1024, hist, g3);
        arrive_wait(lvl + 2, (uint32_t)nch, err, ctrl);
        const BinSplit s3 = find_bin_of_rank_global<1024>(g3, R, lds.scratch);
        R -= s3.above;
        thr = (pre2 << 10) | (uint32_t)s3.bin;
        if (s3.count != R) {
          // More tokens with key thr than places: the lowest positions first.
          uint32_t mine = 0;
#pragma unroll
          for (int u = 0; u < 16; ++u) mine += (((valid >> u) & 1u) && key[u] == thr) ? 1u : 0u;
          uint32_t tot;
          block_exclusive_scan(mine, lds.scratch, tot);
          if (tid == 0) store_coherent(gt + c, tot);
          arrive_wait(lvl + 3, (uint32_t)nch, err, ctrl);
          uint32_t before = 0;
          for (int x = 0; x < c; ++x) before += load_coherent(gt + x);
          take = R > before ? R - before : 0u;
          ties = true;
        }
      }
    }
  }
  MONO_STAMP(8);
  // Selected: every valid token with key > thr, and of those equal to thr
  // all of them, or with ties the first `take` of the request in position
  // order (this thread's share: its lowest equal keys after the tie_rank
  // equal keys of the threads before it).
  uint32_t gt_mask = 0, eq_mask = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    gt_mask |= key[u] > thr ? (1u << u) : 0u;
    eq_mask |= key[u] == thr ? (1u << u) : 0u;
  }
  gt_mask &= valid;
  eq_mask &= valid;
  uint32_t selm = all ? valid : (gt_mask | eq_mask);
  if (ties) {
    uint32_t tot;
    const uint32_t tie_rank = block_exclusive_scan((uint32_t)__popc(eq_mask), lds.scratch, tot);
    uint32_t keep = take > tie_rank ? take - tie_rank : 0u, drop = eq_mask;
    while (drop && keep) {  // the lowest `keep` equal keys stay selected
      drop &= drop - 1u;
      --keep;
    }
    if (!all) selm &= ~drop;
  }
  uint32_t n_sel;
  const uint32_t off = block_exclusive_scan((uint32_t)__popc(selm), lds.scratch, n_sel);
  {
    uint32_t bits = selm, o = off;
    while (bits) {
      const int u = __builtin_ctz(bits);
      bits &= bits - 1u;
      lds.list[o++] = (uint16_t)(16 * tid + u);
    }
  }
  // Output slots: a block of n_sel taken from the token's counter (its value
  // is needed only after the attention), or position j itself when every
  // valid token is selected.  Then this chunk has read every global row it
  // needs; the last chunk to get here clears them after its attention.
  uint32_t base = 0, done_prev = 0;
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    if (!all && n_sel) base = atomicAdd(ctrl + lay.out_cnt + i, n_sel);
    done_prev = atomicAdd(lvl + 4, 1u);
  }

  MONO_STAMP(9);
  const int H = lay.H;
  for (int h = 0; h < H; ++h) {
    const size_t qh = (size_t)i * H + h;
    AttnArgs aa;
    aa.q = a.q + qh * kQHeads * kHeadDim;
    aa.k_pages = a.k_pages;
    aa.v_pages = a.v_pages;
    aa.num_pages = a.num_pages;
    aa.H = H;
    aa.h = h;
    aa.bt_row = nullptr;
    aa.sel_row = nullptr;
    aa.sel_ready = nullptr;
    aa.ctrl = ctrl;
    aa.pos = L - 1;
    aa.e0 = 0;
    aa.e1 = (int)n_sel;
    aa.split = c;
    aa.n_splits = nch;
    aa.scale = a.scale * a.k_scale;
    aa.v_scale = a.v_scale;
    aa.out = a.out + qh * kQHeads * kHeadDim;
    const size_t S = (size_t)lay.part_splits;
    aa.pm = reinterpret_cast<float*>(a.ws + lay.pm) + qh * S * kQHeads;
    aa.pl = reinterpret_cast<float*>(a.ws + lay.pl) + qh * S * kQHeads;
    aa.pacc = reinterpret_cast<float*>(a.ws + lay.pacc) + qh * S * kQHeads * kHeadDim;
    aa.split_cnt = ctrl + lay.attn_cnt + qh;
    aa.err = err;
    aa.llist = (const __attribute__((address_space(3))) uint16_t*)lds.list;
    aa.lptab = (const __attribute__((address_space(3))) int32_t*)lds.ptab;
    aa.tok0 = tok0;
    aa.page0 = p_begin;
    const bool merged = attn_split<Fmt, true>(aa, lds.u.attn);
    // The workgroup that wrote the output is the last to use the split
    // counter, and every chunk's output-slot atomic completed before its
    // split arrived (the wait before the arrival covers it): both counters
    // can start from zero for the next call.
    if (merged && tid == 0) {
      aa.split_cnt[0] = 0u;
      if (h == 0) {
        wait_vmem();
        ctrl[lay.out_cnt + i] = 0u;
      }
    }
    __syncthreads();  // the next head reuses the combine area
  }

  if (tid == 0) {
    lds.scratch[kWaves] = base;
    lds.scratch[kWaves + 1] = done_prev;
  }
  __syncthreads();
  base = lds.scratch[kWaves];
  done_prev = lds.scratch[kWaves + 1];
  {
    int32_t* out = a.sel + (size_t)i * k;
    uint32_t bits = selm, o = off;
    while (bits) {
      const int u = __builtin_ctz(bits);
      bits &= bits - 1u;
      const int j = tok0 + 16 * tid + u;
      const uint32_t slot = all ? (uint32_t)j : base + o;
      ++o;
      if (slot < (uint32_t)k) {
        out[slot] = j;  // read by no item of this launch: plain stores, written back at its end
      } else {
        raise_error(err, kErrSelection);
      }
    }
    if (all && c == 0)
      for (int x = L + tid; x < k; x += kBlock) out[x] = -1;
  }
  if (done_prev == (uint32_t)(nch - 1)) {
    // Every chunk of the request has passed its barriers and read the rows.
    for (int x = tid; x < kHistBins; x += kBlock) {
      g1[x] = 0u;
      g2[x] = 0u;
    }
    for (int x = tid; x < 1024; x += kBlock) g3[x] = 0u;
    if (tid < kLocalMaxChunks) gt[tid] = 0u;
    if (tid < kLvlWords) lvl[tid] = 0u;
    if (exchanged) {  // the exchanged pairs and counts (lds.xc holds every chunk's count)
      uint64_t* xc_all = reinterpret_cast<uint64_t*>(a.ws + lay.xcand) + (size_t)i * kLocalMaxChunks * kExchCap;
      uint32_t* xn_all = reinterpret_cast<uint32_t*>(a.ws + lay.xcnt) + (size_t)i * kLocalMaxChunks;
      for (int cc = 0; cc < nch; ++cc) {
        const uint32_t n_cc = min(lds.xc[cc], (uint32_t)kExchCap);
        for (uint32_t r = (uint32_t)tid; r < n_cc; r += kBlock) xc_all[(size_t)cc * kExchCap + r] = 0ull;
      }
      if (tid < nch) xn_all[tid] = 0u;
    }
  }
}

// Every slice slot of query row i arrives (n_slots in all, whether it held
// scores or not; its outputs complete before it arrives); the last one
// resets the row's counters, resolves the selection and publishes the
// row's attention splits.
template <int TQ>
__device__ __forceinline__ void slice_arrive(const StepArgs& a, const StepLayout& lay, int i, const SelectArgs& sa,
                                             bool valid, bool sliced, BinSplit split, uint32_t n_slots,
                                             StepLds<TQ>& lds, uint32_t* ctrl, uint32_t* err, uint32_t& s_flag,
                                             uint32_t& s_pub) {
  __syncthreads();
  if (thread_index() == 0) {
    s_flag = atomicAdd(ctrl + lay.filter_cnt + i, 1u) == n_slots - 1u;
    if (s_flag) {  // every slice of the row has used its counters
      ctrl[lay.filter_cnt + i] = 0u;
      ctrl[lay.out_cnt + i] = 0u;
      ctrl[lay.cand_cnt + i] = 0u;
    }
  }
  __syncthreads();
  MONO_STAMP(3);
  if (!s_flag) return;
  // Attention items of token i are numbered split-major (split * H + h), so
  // the splits whose candidates are final can be published as one range:
  // the tokens above the threshold bin fill the first output slots before
  // the rest are picked, and their splits run while this workgroup picks.
  const uint32_t H = (uint32_t)lay.H, S = (uint32_t)lay.n_splits;
  const uint32_t first = (uint32_t)i * H * S;
  uint32_t n_early = 0;
  if (valid) {
    // Once the threshold is known, every split is published: those whose
    // candidates are already final as such, the rest gated on the row's
    // ready word, so that they load their q operands and block-table rows
    // while the selection is finished.
    bool published = false;
    resolve_query(sa, lds.resolve, sliced, split, [&](uint32_t n_final) {
      MONO_STAMP(4);
      if (lay.mode != kModeFused) return;
      n_early = n_final >= (uint32_t)lay.k ? S : min(S, n_final / (uint32_t)lay.split_tokens);
      if (n_early) publish(lay, ctrl, kItemAttn, first, n_early * H, err, s_pub);
      __syncthreads();  // the next publication reuses s_pub
      if (n_early < S) publish(lay, ctrl, kItemAttnGated, first + n_early * H, (S - n_early) * H, err, s_pub);
      published = true;
    });
    wait_vmem();
    __syncthreads();
    // The row's selection is complete (every output slot written).
    if (lay.has_sel_ready && thread_index() < lay.H) store_coherent(ctrl + lay.sel_ready + (size_t)i * lay.H + thread_index(), 1u);
    MONO_STAMP(5);
    if (published) return;
  }
  if (lay.mode == kModeFused && n_early < S)
    publish(lay, ctrl, kItemAttn, first + n_early * H, (S - n_early) * H, err, s_pub);
}

template <int TQ, class Fmt>
__device__ __forceinline__ void scan_item(const StepArgs& a, const StepLayout& lay, uint32_t t, StepLds<TQ>& slds,
                                          uint32_t* ctrl, uint32_t* err, uint32_t& s_flag, uint32_t& s_pub) {
  ScanLds<TQ>& lds = slds.scan;
  const int per_b = lay.q_groups * lay.chunks;
  const int b = (int)(t / per_b);
  const int rem = (int)(t % per_b);
  const int qg = rem / lay.chunks, c = rem % lay.chunks;
  const int T = lay.T;
  const int L = a.seq_lens[b];
  // The group's rows: the request's (head, token) pairs u0..u0+tq-1.
  const int u0 = qg * 4;
  const int tq = min(4, lay.G * T - u0);
  // Local filtering (one row per request, every scan item a first-round
  // ticket): the chunk filters its own scores from LDS once the row's
  // histogram is complete, as the row's slice, instead of writing them out
  // and publishing filter items.
  const bool local_filter = TQ == 1 && lay.local_filter;
  const bool valid = L >= T && L <= lay.lcap;
  const int row_i = index_row(lay, b, u0);
  const int n_valid = valid ? window_valid(lay, L - T) : 0;
  const SelectArgs fa = select_args(a, lay, row_i, n_valid, ctrl, err);
  BinSplit split{0, 0u, 0u};
  bool sliced = false;
  if (!valid) {
    if (c == 0 && qg == 0 && thread_index() == 0) raise_error(err, kErrSeqLen);
  } else {
    ScanArgs sa;
    int last = 0;  // position of the group's last-placed token
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int u = u0 + min(m, tq - 1);
      sa.row[m] = index_row(lay, b, u);
      const int pos = L - T + u % T;
      sa.pos[m] = pos - lay.win_lo * kPageTokens;  // scores are indexed from the window's first token
      last = max(last, pos);
    }
    // The group's pages inside the window, relative to its first page.
    const int n_pages = (last + 1 + kPageTokens - 1) / kPageTokens;
    const int n_rel = max(0, min(n_pages, lay.win_hi) - lay.win_lo);
    const int nchunks = (n_rel + lay.chunk_pages - 1) / lay.chunk_pages;
    if (c < nchunks) {
      sa.index_q = a.index_q;
      sa.pages = a.index_pages;
      sa.num_pages = a.num_pages;
      sa.bt_row = a.block_table + (size_t)b * a.bt_stride + lay.win_lo;
      sa.scores = reinterpret_cast<float*>(a.ws + lay.scores);
      sa.ghist = reinterpret_cast<uint32_t*>(a.ws + lay.hist);
      sa.err = err;
      sa.lcap = lay.lcap;
      sa.tq = tq;
      sa.p_begin = c * lay.chunk_pages;
      sa.p_end = min(sa.p_begin + lay.chunk_pages, n_rel);
      if constexpr (TQ == 1) {
        ScanStageLds& st = slds.stage;
        scan_chunk<1, Fmt, true>(sa, st.scan, (lds_f32*)st.scores, (lds_i32w*)st.ptab);
        __syncthreads();
        // The chunk's whole lines of the score row (entries past the
        // row's last valid position hold values no reader uses).
        const uint32_t n_bytes = (uint32_t)(sa.p_end - sa.p_begin) * kPageTokens * 4u;
        auto write_lines = [&]() {
          const __amdgpu_buffer_rsrc_t rsrc =
              buffer_rsrc(sa.scores + (size_t)sa.row[0] * sa.lcap + (size_t)sa.p_begin * kPageTokens, n_bytes);
          const u32x4_t* src = reinterpret_cast<const u32x4_t*>(st.scores);
          for (uint32_t q = (uint32_t)thread_index(); q * 16u < n_bytes; q += kBlock)
            store_coherent_x4(rsrc, q * 16u, src[q]);
        };
        if (local_filter) {
          MONO_STAMP(7);
          if (n_valid > lay.k) {
            // The row's histogram is complete once it counts all n_valid
            // tokens (counts only grow); read until then.
            for (uint32_t spins = 0;; ++spins) {
              uint32_t total;
              split = find_bin_of_rank_global<kHistBins>(fa.ghist, (uint32_t)lay.k, st.scan.hist, &total);
              if (total == (uint32_t)n_valid) break;  // the same in every thread
              if (spins > kMaxSpins) {
                if (thread_index() == 0) wait_ran_out(err, ctrl);
                break;
              }
              __builtin_amdgcn_s_sleep(2);
            }
            MONO_STAMP(6);
            // An overflowing candidate list is resolved from the score row.
            if (split.count > (uint32_t)kCandCap) write_lines();
          }
          const int j0 = sa.p_begin * kPageTokens;
          split = filter_slice<true>(fa, j0, min(j0 + (sa.p_end - sa.p_begin) * kPageTokens, n_valid), slds.filter,
                                     (lds_f32*)st.scores, n_valid > lay.k ? &split : nullptr);
          sliced = true;
        } else {
          write_lines();
        }
      } else {
        scan_chunk<TQ, Fmt>(sa, lds);
      }
      wait_vmem();  // scores and histogram updates are complete before the arrival
      MONO_STAMP(2);
    }
  }
  if (local_filter) {  // every chunk slot of the row arrives as one of its slices
    slice_arrive<TQ>(a, lay, row_i, fa, valid, sliced, split, (uint32_t)lay.chunks, slds, ctrl, err, s_flag, s_pub);
    return;
  }
  // Every chunk slot of the group arrives, with or without work; the last
  // one publishes the selection work of the group's rows.
  __syncthreads();
  if (thread_index() == 0) {
    uint32_t* done = ctrl + lay.scan_done + (size_t)b * lay.q_groups + qg;
    s_flag = atomicAdd(done, 1u) == (uint32_t)(lay.chunks - 1);
    if (s_flag) *done = 0u;  // the last arrival: the counter's last use in this call
  }
  __syncthreads();
  MONO_STAMP(3);
  if (!s_flag) return;
  if (lay.G == 1) {  // the group's rows are consecutive
    const uint32_t q0 = (uint32_t)(b * T + u0);
    if (!lay.select_mode) {
      publish(lay, ctrl, kItemFilter, q0 * (uint32_t)lay.slices, (uint32_t)(tq * lay.slices), err, s_pub);
    } else if (T == 1) {
      select_item<TQ>(a, lay, q0, slds, ctrl, err, s_pub);
    } else {
      publish(lay, ctrl, kItemSelect, q0, (uint32_t)tq, err, s_pub);
    }
  } else {
    for (int m = 0; m < tq; ++m) {
      const uint32_t row = (uint32_t)index_row(lay, b, u0 + m);
      if (!lay.select_mode) {
        publish(lay, ctrl, kItemFilter, row * (uint32_t)lay.slices, (uint32_t)lay.slices, err, s_pub);
      } else {
        publish(lay, ctrl, kItemSelect, row, 1u, err, s_pub);
      }
      __syncthreads();  // the next publication reuses s_pub
    }
  }
}

template <int TQ>
__device__ __forceinline__ void filter_item(const StepArgs& a, const StepLayout& lay, uint32_t u, StepLds<TQ>& lds,
                                            uint32_t* ctrl, uint32_t* err, uint32_t& s_flag, uint32_t& s_pub) {
  const int i = (int)(u / lay.slices), s = (int)(u % lay.slices);
  const int T = lay.T;
  int b, t;
  row_request(lay, i, b, t);
  const int L = a.seq_lens[b];
  const bool valid = L >= T && L <= lay.lcap;  // an invalid length was reported by the scan items
  const int n_valid = window_valid(lay, L - T + t);
  // A query that sees no token of the window still runs slice 0, which
  // writes its -1 padding.
  const int n_slices = valid ? max(1, (n_valid + kSlice - 1) / kSlice) : 0;

  const SelectArgs sa = select_args(a, lay, i, n_valid, ctrl, err);
  BinSplit split{0, 0u, 0u};
  const bool sliced = s < n_slices;
  if (sliced) {
    split = filter_slice(sa, s * kSlice, min((s + 1) * kSlice, n_valid), lds.filter);
    wait_vmem();
    MONO_STAMP(2);
  }
  slice_arrive<TQ>(a, lay, i, sa, valid, sliced, split, (uint32_t)lay.slices, lds, ctrl, err, s_flag, s_pub);
}

template <class Fmt, int kGroups = kPassGroups>
__device__ __forceinline__ void attn_item(const StepArgs& a, const StepLayout& lay, uint32_t v, AttnLds& lds,
                                          uint32_t* ctrl, uint32_t* err, bool gated = false) {
  const int H = lay.H, S = lay.n_splits;
  const int i = (int)(v / (uint32_t)(H * S));
  const int rem = (int)(v % (uint32_t)(H * S));
  const int split = rem / H, h = rem % H;  // split-major (filter_item publishes final splits first)
  const int T = lay.T, b = i / T, t = i % T;
  const int L = a.seq_lens[b];
  if (L < T || L > lay.lcap) {
    if (split == 0 && h == 0 && thread_index() == 0) raise_error(err, kErrSeqLen);
    return;
  }
  const int pos = L - T + t;
  const int list_len = lay.sparse ? lay.k : pos + 1;
  const int n_splits = lay.sparse ? S : (list_len + lay.split_tokens - 1) / lay.split_tokens;
  if (split >= n_splits) return;

  const size_t qh = (size_t)i * H + h;
  AttnArgs aa;
  aa.q = a.q + qh * kQHeads * kHeadDim;
  aa.k_pages = a.k_pages;
  aa.v_pages = a.v_pages;
  aa.num_pages = a.num_pages;
  aa.H = H;
  aa.h = h;
  aa.bt_row = a.block_table + (size_t)b * a.bt_stride;
  aa.sel_row = lay.sparse ? a.sel + (size_t)i * lay.k : nullptr;
  aa.pos = pos;
  aa.e0 = split * lay.split_tokens;
  aa.e1 = min(aa.e0 + lay.split_tokens, list_len);
  aa.split = split;
  aa.n_splits = n_splits;
  aa.scale = a.scale * a.k_scale;
  aa.v_scale = a.v_scale;
  aa.out = a.out + qh * kQHeads * kHeadDim;
  aa.pm = reinterpret_cast<float*>(a.ws + lay.pm) + qh * S * kQHeads;
  aa.pl = reinterpret_cast<float*>(a.ws + lay.pl) + qh * S * kQHeads;
  aa.pacc = reinterpret_cast<float*>(a.ws + lay.pacc) + qh * S * kQHeads * kHeadDim;
  aa.split_cnt = ctrl + lay.attn_cnt + qh;
  aa.err = err;
  aa.sel_ready = gated ? ctrl + lay.sel_ready + qh : nullptr;
  aa.ctrl = ctrl;
  // The workgroup that wrote the output is the last to use the split
  // counter and the ready word of its (row, KV head) (every split arrived
  // before it merged, every gated one after reading the word): both start
  // from zero for the next call.
  if (attn_split<Fmt, false, kGroups>(aa, lds) && thread_index() == 0) {
    if (n_splits > 1) aa.split_cnt[0] = 0u;
    if (lay.has_sel_ready) ctrl[lay.sel_ready + qh] = 0u;
  }
}

// Item sets of the kernel instances: every kind; the chunk-local step's
// clear and chunk-local items (a far smaller program than the instance with
// every item kind, whose code does not fit the instruction cache); the
// attention call's clear and attention items.
enum : int { kSetAll = 0, kSetLocal = 1, kSetAttn = 2 };

template <int TQ, class Fmt, int kSet>
__device__ __forceinline__ void step_body(const StepArgs& a, const StepLayout& lay) {
  constexpr bool kLocal = kSet == kSetLocal;
  static_assert(kSet == kSetAll || TQ == 1, "the chunk-local and attention instances have one query token per group");
  __shared__ std::conditional_t<kLocal, LocalLds, std::conditional_t<kSet == kSetAttn, AttnLds, StepLds<TQ>>> lds;
  __shared__ uint32_t s_item, s_flag, s_clear, s_rec, s_desc, s_pub;
  const int tid = thread_index();
  uint32_t* err = reinterpret_cast<uint32_t*>(a.ws + lay.err);
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(a.ws + lay.ctrl_base);
  MONO_STAMP_GROUP(0);

  // The header records how much of the workspace the previous call left
  // zero.  If that does not cover this layout's zero region (first use, or
  // a larger shape than before), the first tickets clear it and every other
  // item waits for them.  The record only changes after every workgroup has
  // read it, so all workgroups agree.
  if (tid == 0) {
    const uint32_t rec = load_coherent(ctrl + kHdrZeroed);
    s_clear = rec < (uint32_t)lay.zero_units ? lay.n_clear : 0u;
    s_rec = rec;
  }
  __syncthreads();
  const uint32_t n_clear = s_clear;
  // The record stands for this layout exactly (a larger record means bytes
  // past this layout's zero region that this call will dirty).
  const bool record_exact = s_rec == (uint32_t)lay.zero_units;
  const uint32_t n_items = n_clear + lay.n_ready0 + lay.n_queue;

  // A workgroup's first ticket is its index (no start-up rush on the
  // counter); later tickets come from the counter, offset by the grid size,
  // and are taken only when the workgroup is free, so a published item
  // never waits behind a busy workgroup.
  uint32_t t = blockIdx.x;
  for (;;) {
    if (t >= n_items) break;
    if (t < n_clear) {
      MONO_TRACE_ITEM(t, (kTraceClearKind << 24) | t);
      clear_item(lay, t, a.ws, ctrl);
    } else {
      const uint32_t u = t - n_clear;
      if (n_clear) wait_counter(ctrl + kHdrCleared, n_clear, err, ctrl);
      const uint32_t d =
          u < lay.n_ready0 ? ((lay.ready_kind << kKindShift) | u) : wait_slot(ctrl + lay.queue + (u - lay.n_ready0), err, ctrl, s_desc);
      const uint32_t kind = d >> kKindShift, idx = d & kIndexMask;
      MONO_TRACE_ITEM(t, (kind << 24) | idx);
      if constexpr (kLocal) {
        if (kind == kItemScan) local_item<Fmt>(a, lay, idx, lds, ctrl, err);
      } else if constexpr (kSet == kSetAttn) {
        if (kind == kItemAttn) attn_item<Fmt>(a, lay, idx, lds, ctrl, err);
      } else if (kind == kItemScan) {
        scan_item<TQ, Fmt>(a, lay, idx, lds, ctrl, err, s_flag, s_pub);
      } else if (kind == kItemSelect) {
        select_item<TQ>(a, lay, idx, lds, ctrl, err, s_pub);
      } else if (kind == kItemFilter) {
        filter_item<TQ>(a, lay, idx, lds, ctrl, err, s_flag, s_pub);
      } else if (kind == kItemAttn || kind == kItemAttnGated) {
        attn_item<Fmt>(a, lay, idx, lds.attn, ctrl, err, kind == kItemAttnGated);
      }
    }
    MONO_STAMP(1);
    __syncthreads();  // the next item reuses the LDS
    if (n_items <= gridDim.x) break;  // every item was a first ticket: no ticket is left
    if (tid == 0) {
      // Every workgroup ends on exactly one ticket past the last item, so
      // the counter takes n_items increments in all: the last one leaves it
      // at zero for the next call.
      const uint32_t old = atomicAdd(ctrl + kHdrTicket, 1u);
      if (old + 1u == n_items) ctrl[kHdrTicket] = 0u;
      s_item = gridDim.x + old;
    }
    __syncthreads();
    t = s_item;
  }

  // A launch without clear items leaves the control block as it found it:
  // every counter is reset by its last user (each request's chunks, a
  // row's last scan chunk and resolving slice, each token's merging split,
  // the last publisher, each queue slot's consumer, the last ticket).  It
  // may leave the header's zero record as it is only when the record is
  // this layout's own: a record left by a larger layout also covers bytes
  // past this layout's zero region, which this call used as scratch, so
  // the exit below must lower it.  (A wait that ran out has dropped the
  // record already, so the next call clears the region first.)
  MONO_STAMP_GROUP(1);
  if (n_clear == 0u && record_exact) return;
  // Every workgroup has taken its last ticket before it counts itself out,
  // so the last one to leave can reset the control block for the next call
  // and record this layout's zero region as clean.
  if (tid == 0) s_flag = (atomicAdd(ctrl + kHdrExits, 1u) == gridDim.x - 1) ? 1u : 0u;
  __syncthreads();
  if (s_flag) {
    for (size_t x = tid; x < lay.ctrl_words; x += kBlock) ctrl[x] = x == kHdrZeroed ? (uint32_t)lay.zero_units : 0u;
  }
}

template <int TQ, class Fmt, bool kLocal>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void step_kernel(StepArgs a, StepLayout lay) {
  step_body<TQ, Fmt, kLocal ? kSetLocal : kSetAll>(a, lay);
}

template <class Fmt>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(StepArgs a, StepLayout lay) {
  step_body<1, Fmt, kSetAttn>(a, lay);
}

// Compute units of the current device (0 if unknown).
int device_compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 0;
  return cus;
}

// Workgroups that fit on the device at once (cached per device and kernel).
int resident_workgroups(const void* kernel, int variant) {
  static std::mutex mu;
  static int cache[64][kStepVariants] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev][variant] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0) != hipSuccess || per_cu <= 0)
      per_cu = 1;
    cache[dev][variant] = cus * per_cu;
  }
  return cache[dev][variant];
}

}  // namespace

int launch_step(const StepArgs& a, const StepLayout& lay_in, hipStream_t stream, const char* what) {
  const bool f8 = a.fmt == kFmtFp8;
  const void* const kernels[kStepVariants] = {reinterpret_cast<const void*>(&step_kernel<1, Mxfp4Format, false>),
                                              reinterpret_cast<const void*>(&step_kernel<4, Mxfp4Format, false>),
                                              reinterpret_cast<const void*>(&step_kernel<1, Fp8Format, false>),
                                              reinterpret_cast<const void*>(&step_kernel<4, Fp8Format, false>),
                                              reinterpret_cast<const void*>(&step_kernel<1, Mxfp4Format, true>),
                                              reinterpret_cast<const void*>(&step_kernel<1, Fp8Format, true>),
                                              reinterpret_cast<const void*>(&attn_kernel<Mxfp4Format>),
                                              reinterpret_cast<const void*>(&attn_kernel<Fp8Format>)};
  DeviceShape dev{};
  dev.cus = device_compute_units();
  for (int v = 0; v < kStepVariants; ++v) dev.resident[v] = resident_workgroups(kernels[v], v);
  StepLayout lay = lay_in;
  int variant = 0;
  const long grid = plan_step(lay, dev, f8, a.sel_scores != nullptr, &variant, what);
  if (grid <= 0) return (int)grid;  // 0: nothing to do; < 0: refused (message set)
  const int kid = lay.mode == kModeIndex ? (f8 ? kKIndexScanFp8 : kKIndexScan)
                  : lay.mode == kModeAttn  ? (f8 ? kKPaDecodeFp8 : kKPaDecode)
                                           : (f8 ? kKStepFp8 : kKStep);
  const dim3 g((unsigned)grid);
  switch (variant) {
    case 0: MONO_LAUNCH(kid, (step_kernel<1, Mxfp4Format, false>), g, dim3(kBlock), 0, stream, a, lay); break;
    case 1: MONO_LAUNCH(kid, (step_kernel<4, Mxfp4Format, false>), g, dim3(kBlock), 0, stream, a, lay); break;
    case 2: MONO_LAUNCH(kid, (step_kernel<1, Fp8Format, false>), g, dim3(kBlock), 0, stream, a, lay); break;
    case 3: MONO_LAUNCH(kid, (step_kernel<4, Fp8Format, false>), g, dim3(kBlock), 0, stream, a, lay); break;
    case 4: MONO_LAUNCH(kid, (step_kernel<1, Mxfp4Format, true>), g, dim3(kBlock), 0, stream, a, lay); break;
    case 5: MONO_LAUNCH(kid, (step_kernel<1, Fp8Format, true>), g, dim3(kBlock), 0, stream, a, lay); break;
    case 6: MONO_LAUNCH(kid, (attn_kernel<Mxfp4Format>), g, dim3(kBlock), 0, stream, a, lay); break;
    default: MONO_LAUNCH(kid, (attn_kernel<Fp8Format>), g, dim3(kBlock), 0, stream, a, lay); break;
  }
  return check_launch(what);
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate (the allocation-free step
// call).  One array per device holds that call's workspace; the code below
// reaches it only through the address hipGetSymbolAddress returns on each
// device (in host code the array's name is not a device address).
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
constexpr int kScratchInitWords = 1024;  // error word and header (the first 4 KiB)

// Zeroes the error word and the control-block header once per device, so
// the first call clears its own zero region (the header records none).
__global__ void scratch_init_kernel(uint32_t* p) {
  for (int x = threadIdx.x; x < kScratchInitWords; x += blockDim.x) store_coherent(p + x, 0u);
}

// Moves the error bits of the scratch's error word into *dst.
__global__ void scratch_errors_kernel(uint32_t* scratch_err, uint32_t* dst) {
  const uint32_t v = atomicExch(scratch_err, 0u);
  if (v) atomicOr(dst, v);
}

}  // namespace

int noalloc_scratch(hipStream_t stream, uint8_t** ptr) {
  static std::mutex mu;
  static uint8_t* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(MONO_EHIP, "no current HIP device (or device id past %d)", kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess)
      return set_error(MONO_EHIP, "cannot query the stream's capture status");
    if (st != hipStreamCaptureStatusNone)
      return set_error(MONO_EINVAL, "the first call on device %d sets up its scratch and must not be captured", dev);
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return set_error(MONO_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    hipLaunchKernelGGL(scratch_init_kernel, dim3(1), dim3(kBlock), 0, stream, static_cast<uint32_t*>(p));
    if (int rc = check_launch("scratch set-up")) return rc;
    // Later calls may come on other streams: the set-up is complete first.
    const hipError_t es = hipStreamSynchronize(stream);
    if (es != hipSuccess) return set_error(MONO_EHIP, "scratch set-up on device %d: %s", dev, hipGetErrorString(es));
    addr[dev] = static_cast<uint8_t*>(p);
  }
  *ptr = addr[dev];
  return MONO_OK;
}

int launch_scratch_errors(uint8_t* scratch_ptr, size_t err_offset, uint32_t* dst, hipStream_t stream) {
  hipLaunchKernelGGL(scratch_errors_kernel, dim3(1), dim3(1), 0, stream,
                     reinterpret_cast<uint32_t*>(scratch_ptr + err_offset), dst);
  return check_launch("scratch error report");
}

}  // namespace mono

#ifdef MONO_TRACE
// The trace library's record arrays and its two calls.
#include "mono_trace.h"

namespace mono {
__device__ uint64_t g_trace_items[kTraceItems * kTraceStamps];
__device__ uint64_t g_trace_groups[kTraceGroups * kTraceStamps];
}  // namespace mono

extern "C" int mono_trace_clear(void) {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(mono::g_trace_items)) != hipSuccess ||
      hipMemset(p, 0, sizeof(mono::g_trace_items)) != hipSuccess)
    return MONO_EHIP;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(mono::g_trace_groups)) != hipSuccess ||
      hipMemset(p, 0, sizeof(mono::g_trace_groups)) != hipSuccess)
    return MONO_EHIP;
  return hipDeviceSynchronize() == hipSuccess ? MONO_OK : MONO_EHIP;
}

extern "C" int mono_trace_read(uint64_t* items, size_t n_items, uint64_t* groups, size_t n_groups) {
  using mono::kTraceGroups;
  using mono::kTraceItems;
  using mono::kTraceStamps;
  if (n_items > (size_t)kTraceItems * kTraceStamps || n_groups > (size_t)kTraceGroups * kTraceStamps)
    return MONO_EINVAL;
  if (hipDeviceSynchronize() != hipSuccess) return MONO_EHIP;
  if (n_items && hipMemcpyFromSymbol(items, HIP_SYMBOL(mono::g_trace_items), n_items * 8, 0,
                                     hipMemcpyDeviceToHost) != hipSuccess)
    return MONO_EHIP;
  if (n_groups && hipMemcpyFromSymbol(groups, HIP_SYMBOL(mono::g_trace_groups), n_groups * 8, 0,
                                      hipMemcpyDeviceToHost) != hipSuccess)
    return MONO_EHIP;
  return MONO_OK;
}
#endif
