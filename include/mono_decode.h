/*
 * mono_decode.h -- C ABI of the MI355X (gfx950) sparse paged MXFP4 decode library
 * (libmono_decode.so).
 *
 * What the library computes
 * -------------------------
 * One decode step of sparse attention over MXFP4-quantised paged caches:
 *   1. mono_index_score_topk: for every query token, the fp32 dot product of
 *      its bf16 index-q row with every valid dequantised index-K row, then
 *      the k highest-scoring tokens;
 *   2. mono_pa_decode_mxfp4: 16-query-head : 1-KV-head attention (head_dim
 *      128) over the selected tokens, or over every valid token when no
 *      selection is given.
 * mono_sparse_decode_mxfp4 runs both in one launch; mono_insert_mxfp4
 * writes new K, V and index-key rows into the pages.  The *_fp8 calls run
 * the same step over the older build's fp8 caches.
 *
 * Sources.  Page "vllm.models.minimax_m3.amd.ops.mxfp4_pages" (module
 * docstring and mxfp4_page_views) fixes the page: 128 tokens x 64 B of e2m1
 * data (two elements a byte, the even one in the low nibble), then
 * 128 x 4 B of e8m0 scales (one per 32 elements), 8704 B in all, no global
 * scale; K, V and the single index-key head share it, and pa_decode reads
 * [pages, heads, 8704] pools while the index scorers read [pages, 8704].
 * Page "vllm.models.minimax_m3.amd.mono.dispatch" (_step_refusal,
 * _slots_shared) fixes the step tables: one int32 block table, rows
 * bt_stride apart, shared by K, V and the index key; int32 seq_lens; a step
 * decodes T tokens of each of B requests, flattened request-major.  Page
 * "vllm.models.minimax_m3.amd.mono.weights" (_build_cp_qkv) gives the
 * per-rank head shape: 16 query heads of 128 per KV head, one index-q head
 * and one index-key head, each 128 wide.
 *
 * Readings where the pages are silent:
 *   - e2m1 / e8m0 are the OCP Microscaling formats: codes 0..7 are
 *     0, 0.5, 1, 1.5, 2, 3, 4, 6 and 8..15 their negatives; byte e scales
 *     by 2^(e-127), 0xFF is NaN.  Element i of a row uses scale byte i/32.
 *   - Token j of request b is row j%128 of page block_table[b*bt_stride + j/128].
 *   - seq_lens counts every token, the T being decoded included, so query
 *     token t of request b (flat index i = b*T + t) sits at position
 *     pos_i = seq_lens[b] - T + t and sees tokens 0..pos_i.
 *   - The index score is the plain fp32 dot product (no ReLU, weight or
 *     bias); top-k keeps the k highest scores among the valid tokens, ties
 *     to the lower token index, NaN below every number.
 *   - Attention: logits scale * q.k, softmax over the candidates, no sink,
 *     soft-cap or window; an empty candidate set gives a zero output.
 *
 * Conventions of every call
 * -------------------------
 *   - Pointers named *_dev are device pointers (HIP global memory); all
 *     other pointers are host pointers.  bf16 values are passed as uint16_t
 *     bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns: no host synchronisation and no device
 *     allocation, so a sequence of calls can be captured in a HIP graph.
 *     mono_check_device_errors is the one exception (it synchronises).
 *   - The caller owns every buffer, the workspace included.  The library
 *     keeps no state between calls except a thread-local error string.
 *   - Workspaces: ask the *_workspace function for the size; the buffer
 *     must be zero-filled before its first use.  Each call leaves its
 *     counters and histograms zero again and records, in the workspace's
 *     first bytes, how far that zero region reaches; a later call whose
 *     zero region reaches further (another entry point or a larger shape)
 *     clears the difference itself inside its launch.  So one buffer serves
 *     any sequence of calls of any shape that fits it.  Calls that share one
 *     workspace must not overlap in time.
 *   - Return value: MONO_OK (0) or a negative MONO_E* code; on error nothing
 *     was enqueued and mono_last_error() says why.  Nothing aborts.
 *   - Device-side checks: a block-table entry outside [0, num_pages) for a
 *     page that a valid token needs, or seq_lens[b] < T or
 *     seq_lens[b] > bt_stride*128, is not dereferenced; the kernels set a
 *     bit in the workspace's error word instead and the affected outputs
 *     are unspecified.
 */
#ifndef MONO_DECODE_H
#define MONO_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MONO_ABI_VERSION 1

#define MONO_OK 0
#define MONO_EINVAL (-1)  /* bad pointer, size, stride, k, T or B */
#define MONO_ENOTSUP (-2) /* a shape this build does not handle */
#define MONO_ENOSPC (-3)  /* workspace smaller than the *_workspace size */
#define MONO_EHIP (-4)    /* the HIP runtime refused a launch */

/* Device error bits (mono_check_device_errors). */
#define MONO_DEVERR_PAGE_ID 1u     /* block-table entry outside [0, num_pages) */
#define MONO_DEVERR_SEQ_LEN 2u     /* seq_lens[b] < T or > bt_stride*128 */
#define MONO_DEVERR_SELECTION 4u   /* internal selection counts disagreed (a bug; output refused) */
#define MONO_DEVERR_WAIT 8u        /* a bounded wait of one work item on another ran out (a bug) */
#define MONO_DEVERR_SLOT 16u       /* an insert slot at or past num_pages*128 */

/* Geometry of one MXFP4 page (mxfp4_pages page, module docstring). */
#define MONO_PAGE_TOKENS 128
#define MONO_HEAD_DIM 128
#define MONO_PAGE_DATA_BYTES 8192  /* 128 rows x 64 B of packed e2m1 */
#define MONO_PAGE_BYTES 8704       /* + 128 rows x 4 B of e8m0 scales */
#define MONO_Q_HEADS_PER_KV 16

/* ABI version (MONO_ABI_VERSION of the build). */
int mono_abi_version(void);

/* Reason for the last non-zero return on the calling thread ("" if none).
 * The string stays valid until the next call on this thread. */
const char* mono_last_error(void);

/* ---------------------------------------------------------------------------
 * Page packing (mxfp4_pages page, module docstring).
 *
 * mxfp4_pages_pack: codes_dev uint8 [n_pages, 128, 128], one e2m1 code per
 * byte (the high 4 bits are ignored); scales_dev uint8 [n_pages, 128, 4]
 * e8m0; pages_dev uint8 [n_pages, 8704] receives
 *   pages[p][64r + c]        = codes[p][r][2c] | codes[p][r][2c+1] << 4
 *   pages[p][8192 + 4r + g]  = scales[p][r][g].
 * mxfp4_pages_unpack is the exact inverse (codes come out in 0..15).
 * All buffers are contiguous.  n_pages == 0 is a no-op; n_pages < 0 or a
 * NULL pointer with n_pages > 0 gives MONO_EINVAL.
 * ------------------------------------------------------------------------- */
int mxfp4_pages_pack(const uint8_t* codes_dev, const uint8_t* scales_dev, uint8_t* pages_dev,
                     int64_t n_pages, void* stream);
int mxfp4_pages_unpack(const uint8_t* pages_dev, uint8_t* codes_dev, uint8_t* scales_dev,
                       int64_t n_pages, void* stream);

/* Dequantisation of whole pages: out_dev [n_pages, 128, 128].
 * mxfp4_pages_dequant writes fp32: the exact value e2m1(code) * 2^(e-127)
 * rounded to fp32 (round-to-nearest-even; subnormals kept, overflow to inf,
 * e = 0xFF gives NaN, code 8 gives -0.0).
 * mxfp4_pages_dequant_bf16 writes bf16 bit patterns through the very
 * conversion the attention and scoring kernels use, so that conversion can
 * be checked bit for bit against the exact value rounded to bf16. */
int mxfp4_pages_dequant(const uint8_t* pages_dev, float* out_dev, int64_t n_pages, void* stream);
int mxfp4_pages_dequant_bf16(const uint8_t* pages_dev, uint16_t* out_dev, int64_t n_pages,
                             void* stream);

/* ---------------------------------------------------------------------------
 * Index scoring and top-k (the index scorers the mxfp4_pages page names;
 * the rule is the reading above).
 *
 * index_q_dev        bf16 [B*T, 128], query token i = b*T + t.
 * index_pages_dev    uint8 [num_pages, 8704], the single index-key head.
 * block_table_dev    int32 [B, bt_stride], row-contiguous; entries past a
 *                    request's last page are never read.
 * seq_lens_dev       int32 [B]; T <= seq_lens[b] <= bt_stride*128.
 * k                  >= 1.
 * selected_idx_dev   int32 [B*T, k] out: the min(k, pos_i+1) selected token
 *                    positions of query i in any order, then -1 padding.
 * selected_scores_dev  NULL or fp32 [B*T, k] out: the fp32 score of each
 *                    selected token (NaN for padding).
 * ws_dev, ws_bytes   workspace of at least mono_index_score_topk_workspace().
 * ------------------------------------------------------------------------- */
size_t mono_index_score_topk_workspace(int B, int T, int bt_stride, int k);
int mono_index_score_topk(const uint16_t* index_q_dev, const uint8_t* index_pages_dev,
                          int64_t num_pages, const int32_t* block_table_dev, int bt_stride,
                          const int32_t* seq_lens_dev, int B, int T, int k,
                          int32_t* selected_idx_dev, float* selected_scores_dev, void* ws_dev,
                          size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Paged GQA decode attention over MXFP4 K/V pages (the pa_decode the
 * mxfp4_pages page names: [pages, heads, 128, 64] / [pages, heads, 128, 4]
 * views of [pages, heads, 8704] pools).
 *
 * q_dev            bf16 [B*T, kv_heads*16, 128]; query heads 16h..16h+15 read
 *                  KV head h.
 * k_pages_dev, v_pages_dev  uint8 [num_pages, kv_heads, 8704].
 * block_table_dev, bt_stride, seq_lens_dev, B, T: as for the index call.
 * selected_idx_dev NULL: dense, every token 0..pos_i.  Otherwise int32
 *                  [B*T, k]: attention over the listed tokens; entries < 0 or
 *                  > pos_i are skipped; valid entries must be distinct.
 * k                list length (ignored when selected_idx_dev is NULL).
 * scale            logit scale (e.g. 1/sqrt(128)).
 * out_dev          bf16 [B*T, kv_heads*16, 128] out (round-to-nearest-even).
 * ws_dev, ws_bytes workspace of at least mono_pa_decode_workspace() for the
 *                  same (B, T, kv_heads, bt_stride, k, sparse) arguments.
 * ------------------------------------------------------------------------- */
size_t mono_pa_decode_workspace(int B, int T, int kv_heads, int bt_stride, int k, int sparse);
int mono_pa_decode_mxfp4(const uint16_t* q_dev, const uint8_t* k_pages_dev,
                         const uint8_t* v_pages_dev, int64_t num_pages, int kv_heads,
                         const int32_t* block_table_dev, int bt_stride,
                         const int32_t* seq_lens_dev, int B, int T,
                         const int32_t* selected_idx_dev, int k, float scale, uint16_t* out_dev,
                         void* ws_dev, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * One sparse decode step: index scores and top-k (as mono_index_score_topk)
 * followed by attention over the selected tokens (as mono_pa_decode_mxfp4
 * with that selection), in a single launch.  The attention of a query token
 * starts as soon as its own selection is complete, while other query tokens
 * are still being scored.  This composes the two operations the
 * mxfp4_pages page names (index top-k, then the pa_decode gather over the
 * chosen tokens); the results equal those of the two calls in sequence.
 * With T = 1 and rows that fit (at most 16 chunks of 32 pages per request,
 * one workgroup per chunk, all resident at once), the launch runs
 * chunk-local: the chunks of a request exchange histogram counts and the
 * candidates of the threshold bin through the workspace, and each attends
 * over its own share of the selection.  The selected set is the same; the
 * order of the positions in a row may differ.  The workspace then also
 * holds, per query token, 16 exchange regions of 2048 (key, position)
 * pairs (256 KiB), included in mono_sparse_decode_workspace().
 *
 * index_q_dev, index_pages_dev   as for mono_index_score_topk.
 * q_dev, k_pages_dev, v_pages_dev, kv_heads, scale, out_dev   as for
 *                  mono_pa_decode_mxfp4.  The index pool and the K/V pools
 *                  share num_pages and the block table.
 * selected_idx_dev int32 [B*T, k] out: the selection (as the index call).
 * ws_dev, ws_bytes workspace of at least mono_sparse_decode_workspace() for
 *                  the same (B, T, kv_heads, bt_stride, k).
 * ------------------------------------------------------------------------- */
size_t mono_sparse_decode_workspace(int B, int T, int kv_heads, int bt_stride, int k);
int mono_sparse_decode_mxfp4(const uint16_t* index_q_dev, const uint8_t* index_pages_dev,
                             const uint16_t* q_dev, const uint8_t* k_pages_dev,
                             const uint8_t* v_pages_dev, int64_t num_pages, int kv_heads,
                             const int32_t* block_table_dev, int bt_stride,
                             const int32_t* seq_lens_dev, int B, int T, int k, float scale,
                             int32_t* selected_idx_dev, uint16_t* out_dev, void* ws_dev,
                             size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * mono_sparse_decode_mxfp4 for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument.  Its workspace is a static device
 * array of MONO_NOALLOC_SCRATCH_BYTES that the library holds on every
 * device it runs on until the process ends.  The call allocates nothing and
 * calls no allocating routine.
 *
 * Arguments, results and errors are those of mono_sparse_decode_mxfp4,
 * except:
 *   - a shape whose workspace (mono_sparse_decode_workspace) exceeds
 *     MONO_NOALLOC_SCRATCH_BYTES gives MONO_ENOSPC;
 *   - err_dev: NULL, or a device uint32 word into which the device error
 *     bits (MONO_DEVERR_*) this call raised are OR-ed (by a second small
 *     launch on the same stream); the scratch's own error word is cleared.
 *   - The first call on a device sets the scratch up (zeroes its header)
 *     and synchronises `stream` once; it is refused (MONO_EINVAL) while
 *     `stream` is being captured.  Later calls only enqueue work.
 * All calls on one device share its scratch, which keeps the last call's
 * contents (each call leaves what must start at zero zero again): calls
 * that overlap in time on one device race and give unspecified results.
 * ------------------------------------------------------------------------- */
#define MONO_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int mono_sparse_decode_mxfp4_noalloc(const uint16_t* index_q_dev, const uint8_t* index_pages_dev,
                                     const uint16_t* q_dev, const uint8_t* k_pages_dev,
                                     const uint8_t* v_pages_dev, int64_t num_pages, int kv_heads,
                                     const int32_t* block_table_dev, int bt_stride,
                                     const int32_t* seq_lens_dev, int B, int T, int k, float scale,
                                     int32_t* selected_idx_dev, uint16_t* out_dev, uint32_t* err_dev,
                                     void* stream);

/* ---------------------------------------------------------------------------
 * Indexer context parallelism, emulated on one GPU.  Page
 * "vllm.models.minimax_m3.amd.mono.weights", _build_cp_qkv: every rank keeps
 * all ranks' index-q heads, so rank r can score its share of every
 * sequence's index pages for all heads; each head's candidates then go to
 * the head's owner, which keeps its top-k.  Readings: shard r of G owns
 * block-table columns [r*c, min(W, (r+1)*c)), c = ceil(W/G); a shard emits
 * per query token the top-k (position, score) pairs among its tokens that
 * the query sees, by the index call's rule; the owner merges the G lists by
 * the same rule.  The merged selection equals the index call's.
 *
 * mono_index_score_topk_window: mono_index_score_topk (same arguments and
 * workspace) restricted to the tokens of block-table columns
 * [page_lo, page_hi) (0 <= page_lo < page_hi <= bt_stride).
 * selected_idx_dev receives absolute token positions; a query that sees no
 * token of the window gets a row of -1.  selected_scores_dev should be given
 * (the merge needs the scores).
 *
 * mono_topk_merge: cand_idx_dev int32 [G, N, k_in] (positions, < 0 = empty
 * slot) and cand_scores_dev fp32 [G, N, k_in] -> out_idx_dev int32
 * [N, k_out]: the min(k_out, candidates) best by the index call's rule
 * (higher score, ties to the lower position, NaN last), in any order, then
 * -1 padding; out_scores_dev (NULL or fp32 [N, k_out]) their scores, NaN
 * padding.  A position must not appear in two lists.  G * k_in <= 8192
 * (else MONO_ENOTSUP).  No workspace.
 * ------------------------------------------------------------------------- */
int mono_index_score_topk_window(const uint16_t* index_q_dev, const uint8_t* index_pages_dev,
                                 int64_t num_pages, const int32_t* block_table_dev, int bt_stride,
                                 const int32_t* seq_lens_dev, int B, int T, int k, int page_lo,
                                 int page_hi, int32_t* selected_idx_dev,
                                 float* selected_scores_dev, void* ws_dev, size_t ws_bytes,
                                 void* stream);
int mono_topk_merge(const int32_t* cand_idx_dev, const float* cand_scores_dev, int G, int64_t N,
                    int k_in, int k_out, int32_t* out_idx_dev, float* out_scores_dev,
                    void* stream);

/* mono_indexer_cp_topk: the whole emulation in one call, with every head
 * of a shard scored from one read of its window.
 *
 * index_q_dev        bf16 [heads, B*T, 128]: every rank's index-q head (row
 *                    (h, b*T + t)); heads in [1, 64].
 * index_pages_dev .. seq_lens_dev, B, T, k: as mono_index_score_topk.
 * shards             G >= 1: shard r owns block-table columns
 *                    [r*c, min(bt_stride, (r+1)*c)), c = ceil(bt_stride/G);
 *                    shards whose window starts past the table are empty
 *                    and skipped.  (non-empty shards) * k <= 8192, else
 *                    MONO_ENOTSUP.
 * selected_idx_dev   int32 [heads, B*T, k] out: each head's top-k positions
 *                    (any order within a row, -1 padding), equal to the
 *                    index call's selection for that head.
 * ws_dev, ws_bytes   workspace of at least mono_indexer_cp_topk_workspace()
 *                    (256-byte aligned): the index workspace, then the
 *                    shards' candidate lists.
 * Enqueues one index launch per non-empty shard, then the merge; errors as
 * mono_index_score_topk. */
size_t mono_indexer_cp_topk_workspace(int B, int T, int heads, int bt_stride, int k, int shards);
int mono_indexer_cp_topk(const uint16_t* index_q_dev, const uint8_t* index_pages_dev,
                         int64_t num_pages, const int32_t* block_table_dev, int bt_stride,
                         const int32_t* seq_lens_dev, int B, int T, int heads, int k, int shards,
                         int32_t* selected_idx_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The same step over fp8 caches (the older build's format: page
 * "vllm.models.minimax_m3.amd.mono.weights", SparseMoeLayer, names an fp8
 * index cache [blocks, block, head_dim] with shared block ids and the KV
 * cache scales the layer's attention holds; page
 * "vllm.models.minimax_m3.amd.mono.dispatch", _config_refusal, requires fp8
 * KV and index caches).
 *
 * Readings where the pages only say "fp8":
 *   - elements are OCP FP8 E4M3 (e4m3fn): bias 7, no infinities, 0x7F and
 *     0xFF are NaN, largest value 448;
 *   - a page is 128 tokens x 128 elements, one byte each, row-major (element
 *     i of token row r at byte 128*r + i): MONO_FP8_PAGE_BYTES = 16384;
 *     K/V pools are [num_pages, kv_heads, 16384], the index pool
 *     [num_pages, 16384];
 *   - K and V each carry one fp32 tensor scale: a K element is
 *     e4m3 * k_scale, a V element e4m3 * v_scale.  The index cache has no
 *     scale (its scores are plain dot products with the e4m3 values).
 *
 * Every argument, rule and error is that of the MXFP4 call of the same name
 * (the workspace functions above serve both), except that the pools are fp8
 * and the attention calls take k_scale and v_scale (finite, > 0), which
 * multiply the logits and the output.  fp8_pages_dequant_bf16 converts
 * whole pages [n_pages, 16384] to bf16 [n_pages, 128, 128] through the
 * kernels' own conversion (exact: every e4m3 value is a bf16 value).
 * ------------------------------------------------------------------------- */
#define MONO_FP8_PAGE_BYTES 16384
int mono_index_score_topk_fp8(const uint16_t* index_q_dev, const uint8_t* index_pages_dev,
                              int64_t num_pages, const int32_t* block_table_dev, int bt_stride,
                              const int32_t* seq_lens_dev, int B, int T, int k,
                              int32_t* selected_idx_dev, float* selected_scores_dev, void* ws_dev,
                              size_t ws_bytes, void* stream);
int mono_pa_decode_fp8(const uint16_t* q_dev, const uint8_t* k_pages_dev,
                       const uint8_t* v_pages_dev, int64_t num_pages, int kv_heads,
                       const int32_t* block_table_dev, int bt_stride, const int32_t* seq_lens_dev,
                       int B, int T, const int32_t* selected_idx_dev, int k, float scale,
                       float k_scale, float v_scale, uint16_t* out_dev, void* ws_dev,
                       size_t ws_bytes, void* stream);
int mono_sparse_decode_fp8(const uint16_t* index_q_dev, const uint8_t* index_pages_dev,
                           const uint16_t* q_dev, const uint8_t* k_pages_dev,
                           const uint8_t* v_pages_dev, int64_t num_pages, int kv_heads,
                           const int32_t* block_table_dev, int bt_stride,
                           const int32_t* seq_lens_dev, int B, int T, int k, float scale,
                           float k_scale, float v_scale, int32_t* selected_idx_dev,
                           uint16_t* out_dev, void* ws_dev, size_t ws_bytes, void* stream);
int fp8_pages_dequant_bf16(const uint8_t* pages_dev, uint16_t* out_dev, int64_t n_pages,
                           void* stream);

/* ---------------------------------------------------------------------------
 * Cache insert: quantise bf16 rows to MXFP4 and write them into the pages
 * through a slot mapping.  Page "vllm.models.minimax_m3.amd.mono.dispatch"
 * (_slots_shared, _step_refusal): K/V and the index key are written through
 * one int64 slot mapping with pages of 128 tokens, shared by both caches;
 * the mxfp4_pages page names the writer and fixes the page.  Slot s is row
 * s%128 of page s/128 of every written cache.
 *
 * Rounding (a reading: the pages print no rule) is the OCP Microscaling
 * v1.0 conversion, per 32-element block: scale byte
 * clamp(floor(log2 max|v|) - 2 + 127, 0, 254); element code = the e2m1
 * value nearest v / 2^(byte-127), ties to the even code, magnitudes above 6
 * saturating to 6, sign in bit 3 (-0.0 gives code 8); an all-zero block
 * has byte 0; a block holding NaN or +-inf gets byte 0xFF and codes 0.
 * The scale byte comes from integer arithmetic on the bf16 exponent
 * fields; each pair of elements is converted by the gfx950 scaled fp4
 * conversion with the fp32 scale 2^(byte-127), which rounds to nearest,
 * ties to even, and saturates at 6 exactly as above.
 *
 * k_rows_dev, v_rows_dev  bf16 [n, kv_heads, 128]; index_rows_dev bf16
 *                  [n, 128].  Each may be NULL together with its pool, and
 *                  that cache is not written.
 * slots_dev        int64 [n]; a negative slot skips token t (padding).  A
 *                  slot at or past num_pages*128 is not written and sets
 *                  MONO_DEVERR_SLOT in *err_dev.  Non-negative slots must be
 *                  distinct (else which row lands is unspecified).
 * k_pages_dev, v_pages_dev  uint8 [num_pages, kv_heads, 8704];
 * index_pages_dev  uint8 [num_pages, 8704].  Only the written rows' 64 data
 *                  bytes and 4 scale bytes change.
 * err_dev          uint32 device word; error bits are OR-ed into it.  The
 *                  first word of any workspace above serves, so that
 *                  mono_check_device_errors reads and clears it.
 * n == 0 is a no-op.  Rows and pages need 16-byte alignment.
 * ------------------------------------------------------------------------- */
int mono_insert_mxfp4(const uint16_t* k_rows_dev, const uint16_t* v_rows_dev,
                      const uint16_t* index_rows_dev, const int64_t* slots_dev, int64_t n,
                      int kv_heads, uint8_t* k_pages_dev, uint8_t* v_pages_dev,
                      uint8_t* index_pages_dev, int64_t num_pages, uint32_t* err_dev,
                      void* stream);

/* ---------------------------------------------------------------------------
 * Per-kernel timing, for benchmarks and profiling only (not for graph capture).
 *
 * mono_profile_start(capacity): from now on every kernel the library launches
 * is bracketed by a pair of HIP events recorded on its stream, for at most
 * `capacity` launches (later launches are not timed).  Creates 2*capacity
 * events.  MONO_EINVAL if already started or capacity is out of [1, 2^20].
 * mono_profile_stop(total_ms, launches, n): waits for the recorded events and
 * writes, for kernel ids 0..n-1, the summed milliseconds and the number of
 * timed launches (host arrays of n entries), then destroys the events.
 * Returns the number of kernel ids the library has (MONO_NUM_KERNELS) or a
 * negative code.  mono_kernel_name(id) is the kernel's name ("" if unknown).
 * ------------------------------------------------------------------------- */
#define MONO_NUM_KERNELS 17
int mono_profile_start(int capacity);
int mono_profile_stop(double* total_ms, int* launches, int n);
const char* mono_kernel_name(int id);

/* ---------------------------------------------------------------------------
 * Read-bandwidth references, for benchmarks only: how fast the device reads
 * MXFP4 pages (mxfp4_pages page: 8704-B pages, 128 x 64 data bytes then
 * 128 x 4 scale bytes) when it has nothing else to do.
 *
 * mode 0: every byte of pages_dev [n_pages, 8704] in address order, 16 B per
 *         lane per load;
 * mode 1: the pages page_ids_dev[0..n_pages) (int32 ids into pages_dev),
 *         each read as the index scan reads it (per 16-row tile, 16 data
 *         bytes and one scale byte per lane).
 * `grid` workgroups of 256 threads each read a contiguous share and store
 * one word to sink_dev[0..grid).  Loads carry the non-temporal hint.
 * MONO_EINVAL for a bad mode, size, grid (1..65536) or pointer.
 * ------------------------------------------------------------------------- */
int mono_bench_read(const uint8_t* pages_dev, const int32_t* page_ids_dev, int64_t n_pages, int mode,
                    int grid, uint32_t* sink_dev, void* stream);

/* ---------------------------------------------------------------------------
 * The index scan on the matrix cores against the same scan on the vector
 * ALUs, for benchmarks only.  Workgroup (b, c) scores pages
 * [c*chunk_pages, ...) of request b's block-table row for query row b of
 * index_q_dev (bf16 [B, 128]; one query token per request, at position
 * seq_lens[b] - 1), keeps the scores in LDS and adds their histogram over
 * the top 11 score-key bits to hist_dev[b] (uint32 [B, 2048], accumulated:
 * the caller zeroes it).  Scores are the mxfp4_pages page's dot products of
 * the query with the exactly dequantised token rows.
 *   variant 0: the step's scan (bf16 MFMA 16x16x32);
 *   variant 1: v_dot2_f32_bf16 on the VALU, two lanes per token row.
 * chunk_pages in [1, 32].  err_dev: MONO_DEVERR_PAGE_ID on a bad page id,
 * MONO_DEVERR_SEQ_LEN for a length outside [1, bt_stride*128] (that request
 * is skipped).
 * MONO_EINVAL for bad sizes, variant or pointers.
 * ------------------------------------------------------------------------- */
int mono_bench_scan(const uint16_t* index_q_dev, const uint8_t* index_pages_dev, int64_t num_pages,
                    const int32_t* block_table_dev, int bt_stride, const int32_t* seq_lens_dev, int B,
                    int chunk_pages, int variant, uint32_t* hist_dev, uint32_t* err_dev, void* stream);

/* Debug/test only.  Waits for `stream`, then returns the device error bits
 * (MONO_DEVERR_*) accumulated in the workspace and clears them, or a
 * negative MONO_E* code.  ws_dev is a workspace of any call above. */
int mono_check_device_errors(void* ws_dev, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MONO_DECODE_H */
