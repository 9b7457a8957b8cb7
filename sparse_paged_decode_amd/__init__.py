"""MI355X (gfx950) sparse paged MXFP4 decode attention.

The compute lives in ``libmono_decode.so`` (hand-written HIP kernels behind
a C ABI, declared in ``include/mono_decode.h``); this package is its thin
Python binding.  PyTorch supplies device memory and streams only.

Step of the method (page *vllm.models.minimax_m3.amd.ops.mxfp4_pages*:
MXFP4 K, V and index-key pages; page *vllm.models.minimax_m3.amd.mono.dispatch*:
pure-decode steps over one shared block table):

    sel = mono_index_score_topk(index_q, index_pages, block_table, seq_lens, k, T=T)
    out = mono_pa_decode_mxfp4(q, k_pages, v_pages, block_table, seq_lens, sel, scale, T=T)

or both in one launch:

    out, sel = mono_sparse_decode_mxfp4(index_q, index_pages, q, k_pages, v_pages,
                                        block_table, seq_lens, k, scale, T=T)

The same step over the older build's fp8 (e4m3) caches, with per-tensor K/V
scales: mono_index_score_topk_fp8, mono_pa_decode_fp8, mono_sparse_decode_fp8.

Indexer context parallelism, emulated on one GPU (G page-window shard scans
of all index heads, then a merge of each head's candidates):
indexer_cp_topk, built on mono_index_score_topk(page_window=...) and
mono_topk_merge.

Callers that cannot allocate device memory (graph capture, serving loops)
use mono_sparse_decode_mxfp4_noalloc: the same step with the library's
static per-device scratch in place of a workspace.

New tokens' K, V and index-key rows enter the pages through the int64 slot
mapping (dispatch page, _slots_shared):

    mono_insert_mxfp4(slots, k_rows=k, v_rows=v, index_rows=ik,
                      k_pages=k_pages, v_pages=v_pages, index_pages=index_pages)
"""

from ._binding import (  # noqa: F401
    DEVERR_PAGE_ID,
    DEVERR_SELECTION,
    DEVERR_SLOT,
    DEVERR_SEQ_LEN,
    DEVERR_WAIT,
    EXPORTED_SYMBOLS,
    FP8_PAGE_BYTES,
    HEAD_DIM,
    KernelTimer,
    MONO_EHIP,
    MONO_EINVAL,
    MONO_ENOSPC,
    MONO_ENOTSUP,
    MONO_OK,
    NOALLOC_SCRATCH_BYTES,
    PAGE_BYTES,
    PAGE_TOKENS,
    Q_HEADS_PER_KV,
    MonoError,
    Workspace,
    bench_read,
    bench_scan,
    check_device_errors,
    cp_shard_windows,
    fp8_pages_dequant_bf16,
    index_score_topk_workspace_bytes,
    indexer_cp_topk,
    load_library,
    mono_index_score_topk,
    mono_index_score_topk_fp8,
    mono_insert_mxfp4,
    mono_pa_decode_fp8,
    mono_pa_decode_mxfp4,
    mono_sparse_decode_fp8,
    mono_sparse_decode_mxfp4,
    mono_sparse_decode_mxfp4_noalloc,
    mono_topk_merge,
    mxfp4_page_views,
    mxfp4_pages_dequant,
    mxfp4_pages_dequant_bf16,
    mxfp4_pages_pack,
    mxfp4_pages_unpack,
    pa_decode_workspace_bytes,
    sparse_decode_workspace_bytes,
)
from .build import LIB_PATH  # noqa: F401
