"""ctypes binding of libmono_decode.so (argument marshalling only).

Every computation happens in the library's HIP kernels; this module checks
tensor arguments, takes device pointers and the current HIP stream from
PyTorch, and raises on a non-zero return code.  If the library is missing or
cannot be loaded, every call raises: there is no fallback path.

Argument checks follow the pages: ``mxfp4_page_views`` on the page
*vllm.models.minimax_m3.amd.ops.mxfp4_pages* (uint8, last dim 8704, unit
byte stride) and ``_step_refusal`` on the page
*vllm.models.minimax_m3.amd.mono.dispatch* (int32 tables, a row-contiguous
block table, tables at least as long as the batch, a token count divisible
by the tokens per request).
"""

import ctypes
import math
import os

import torch

from .build import LIB_PATH

PAGE_TOKENS = 128
HEAD_DIM = 128
DATA_BYTES = 64
SCALE_BYTES = 4
PAGE_BYTES = PAGE_TOKENS * (DATA_BYTES + SCALE_BYTES)  # 8704
FP8_PAGE_BYTES = PAGE_TOKENS * HEAD_DIM  # 16384: the older build's fp8 (e4m3) pages
Q_HEADS_PER_KV = 16

MONO_OK = 0
MONO_EINVAL = -1
MONO_ENOTSUP = -2
MONO_ENOSPC = -3
MONO_EHIP = -4

DEVERR_PAGE_ID = 1
DEVERR_SEQ_LEN = 2
DEVERR_SELECTION = 4
DEVERR_WAIT = 8
DEVERR_SLOT = 16

EXPORTED_SYMBOLS = (
    "mono_abi_version",
    "mono_last_error",
    "mxfp4_pages_pack",
    "mxfp4_pages_unpack",
    "mxfp4_pages_dequant",
    "mxfp4_pages_dequant_bf16",
    "mono_index_score_topk_workspace",
    "mono_index_score_topk",
    "mono_pa_decode_workspace",
    "mono_pa_decode_mxfp4",
    "mono_sparse_decode_workspace",
    "mono_sparse_decode_mxfp4",
    "mono_sparse_decode_mxfp4_noalloc",
    "mono_insert_mxfp4",
    "mono_index_score_topk_fp8",
    "mono_index_score_topk_window",
    "mono_topk_merge",
    "mono_indexer_cp_topk_workspace",
    "mono_indexer_cp_topk",
    "mono_pa_decode_fp8",
    "mono_sparse_decode_fp8",
    "fp8_pages_dequant_bf16",
    "mono_check_device_errors",
    "mono_bench_read",
    "mono_bench_scan",
    "mono_profile_start",
    "mono_profile_stop",
    "mono_kernel_name",
)


class MonoError(RuntimeError):
    """A non-zero return code of libmono_decode.so."""

    def __init__(self, code, message):
        super().__init__(f"[{code}] {message}")
        self.code = code


_lib = None


def load_library(path=LIB_PATH):
    """Load libmono_decode.so and declare its signatures (cached)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run sparse_paged_decode_amd.build.build() "
            "(or __graft_entry__.build()) first"
        )
    lib = ctypes.CDLL(path)
    P, I, I64, SZ, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "mono_abi_version": (I, []),
        "mono_last_error": (ctypes.c_char_p, []),
        "mxfp4_pages_pack": (I, [P, P, P, I64, P]),
        "mxfp4_pages_unpack": (I, [P, P, P, I64, P]),
        "mxfp4_pages_dequant": (I, [P, P, I64, P]),
        "mxfp4_pages_dequant_bf16": (I, [P, P, I64, P]),
        "mono_index_score_topk_workspace": (SZ, [I, I, I, I]),
        "mono_index_score_topk": (I, [P, P, I64, P, I, P, I, I, I, P, P, P, SZ, P]),
        "mono_pa_decode_workspace": (SZ, [I, I, I, I, I, I]),
        "mono_pa_decode_mxfp4": (I, [P, P, P, I64, I, P, I, P, I, I, P, I, F, P, P, SZ, P]),
        "mono_sparse_decode_workspace": (SZ, [I, I, I, I, I]),
        "mono_sparse_decode_mxfp4": (I, [P, P, P, P, P, I64, I, P, I, P, I, I, I, F, P, P, P, SZ, P]),
        "mono_sparse_decode_mxfp4_noalloc": (I, [P, P, P, P, P, I64, I, P, I, P, I, I, I, F, P, P, P, P]),
        "mono_insert_mxfp4": (I, [P, P, P, P, I64, I, P, P, P, I64, P, P]),
        "mono_index_score_topk_fp8": (I, [P, P, I64, P, I, P, I, I, I, P, P, P, SZ, P]),
        "mono_index_score_topk_window": (I, [P, P, I64, P, I, P, I, I, I, I, I, P, P, P, SZ, P]),
        "mono_topk_merge": (I, [P, P, I, I64, I, I, P, P, P]),
        "mono_indexer_cp_topk_workspace": (SZ, [I, I, I, I, I, I]),
        "mono_indexer_cp_topk": (I, [P, P, I64, P, I, P, I, I, I, I, I, P, P, SZ, P]),
        "mono_pa_decode_fp8": (I, [P, P, P, I64, I, P, I, P, I, I, P, I, F, F, F, P, P, SZ, P]),
        "mono_sparse_decode_fp8": (I, [P, P, P, P, P, I64, I, P, I, P, I, I, I, F, F, F, P, P, P, SZ, P]),
        "fp8_pages_dequant_bf16": (I, [P, P, I64, P]),
        "mono_check_device_errors": (I, [P, P]),
        "mono_bench_read": (I, [P, P, I64, I, I, P, P]),
        "mono_bench_scan": (I, [P, P, I64, P, I, P, I, I, I, P, P, P]),
        "mono_profile_start": (I, [I]),
        "mono_profile_stop": (I, [P, P, I]),
        "mono_kernel_name": (ctypes.c_char_p, [I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc):
    if rc != MONO_OK:
        msg = _lib.mono_last_error().decode(errors="replace")
        raise MonoError(rc, msg)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _on_gpu(*ts):
    dev = ts[0].device
    for t in ts:
        _need(t.is_cuda and t.device == dev, "all tensors must be on the same GPU")
    return dev


# --- page views (zero-copy) -------------------------------------------------------


def mxfp4_page_views(pages):
    """(data, scale) zero-copy views of uint8 pages ``[..., 8704]``.

    The page geometry of the mxfp4_pages page (module docstring and
    ``mxfp4_page_views``): bytes 0..8191 of a page are 128 rows of 64 packed
    e2m1 bytes and bytes 8192..8703 are 128 rows of 4 e8m0 bytes.  So the
    data view is the first 8192 bytes of the last axis split into
    ``[..., 128, 64]`` and the scale view the last 512 split into
    ``[..., 128, 4]``; leading dims and strides are those of ``pages``.
    Raises ValueError for a dtype other than uint8, a last dim other than
    8704 or bytes of a page that are not adjacent.
    """
    if pages.dtype != torch.uint8:
        raise ValueError(f"page views need uint8 bytes, not {pages.dtype}")
    if pages.dim() < 1 or pages.shape[-1] != PAGE_BYTES:
        raise ValueError(f"the last axis must be one {PAGE_BYTES}-byte page; shape is {tuple(pages.shape)}")
    if pages.stride(-1) != 1:
        raise ValueError(f"the bytes of a page must be adjacent (last-axis stride {pages.stride(-1)}, not 1)")
    data_bytes = PAGE_TOKENS * DATA_BYTES
    data = pages.narrow(-1, 0, data_bytes).unflatten(-1, (PAGE_TOKENS, DATA_BYTES))
    scale = pages.narrow(-1, data_bytes, PAGE_TOKENS * SCALE_BYTES).unflatten(-1, (PAGE_TOKENS, SCALE_BYTES))
    return data, scale


def _check_pages(pages, name, ndim, page_bytes=None):
    page_bytes = PAGE_BYTES if page_bytes is None else page_bytes
    _need(pages.dtype == torch.uint8, f"{name} must be uint8, got {pages.dtype}")
    _need(pages.dim() == ndim and pages.shape[-1] == page_bytes, f"{name} must be [{'..., ' * (ndim - 1)}{page_bytes}]")
    _need(pages.is_contiguous(), f"{name} must be contiguous")


# --- packing and dequantisation ----------------------------------------------------


def mxfp4_pages_pack(codes, scales, out=None):
    """uint8 codes ``[n, 128, 128]`` + e8m0 scales ``[n, 128, 4]`` -> pages ``[n, 8704]``."""
    load_library()
    _need(codes.dtype == torch.uint8 and codes.dim() == 3 and tuple(codes.shape[1:]) == (128, 128), "codes: uint8 [n,128,128]")
    n = codes.shape[0]
    _need(scales.dtype == torch.uint8 and tuple(scales.shape) == (n, 128, 4), "scales: uint8 [n,128,4]")
    _need(codes.is_contiguous() and scales.is_contiguous(), "codes and scales must be contiguous")
    dev = _on_gpu(codes, scales)
    if out is None:
        out = torch.empty((n, PAGE_BYTES), dtype=torch.uint8, device=dev)
    _check_pages(out, "out", 2)
    _need(out.shape[0] == n, "out must have n pages")
    _check(_lib.mxfp4_pages_pack(_ptr(codes), _ptr(scales), _ptr(out), n, _stream(dev)))
    return out


def mxfp4_pages_unpack(pages):
    """pages ``[n, 8704]`` -> (codes ``[n, 128, 128]``, scales ``[n, 128, 4]``)."""
    load_library()
    _check_pages(pages, "pages", 2)
    dev = _on_gpu(pages)
    n = pages.shape[0]
    codes = torch.empty((n, 128, 128), dtype=torch.uint8, device=dev)
    scales = torch.empty((n, 128, 4), dtype=torch.uint8, device=dev)
    _check(_lib.mxfp4_pages_unpack(_ptr(pages), _ptr(codes), _ptr(scales), n, _stream(dev)))
    return codes, scales


def mxfp4_pages_dequant(pages):
    """pages ``[n, 8704]`` -> exact fp32 values ``[n, 128, 128]``."""
    load_library()
    _check_pages(pages, "pages", 2)
    dev = _on_gpu(pages)
    out = torch.empty((pages.shape[0], 128, 128), dtype=torch.float32, device=dev)
    _check(_lib.mxfp4_pages_dequant(_ptr(pages), _ptr(out), pages.shape[0], _stream(dev)))
    return out


def mxfp4_pages_dequant_bf16(pages):
    """pages ``[n, 8704]`` -> bf16 values ``[n, 128, 128]`` via the kernels' conversion."""
    load_library()
    _check_pages(pages, "pages", 2)
    dev = _on_gpu(pages)
    out = torch.empty((pages.shape[0], 128, 128), dtype=torch.bfloat16, device=dev)
    _check(_lib.mxfp4_pages_dequant_bf16(_ptr(pages), _ptr(out), pages.shape[0], _stream(dev)))
    return out


def fp8_pages_dequant_bf16(pages):
    """fp8 pages ``[n, 16384]`` -> bf16 values ``[n, 128, 128]`` via the kernels' conversion."""
    load_library()
    _check_pages(pages, "pages", 2, FP8_PAGE_BYTES)
    dev = _on_gpu(pages)
    out = torch.empty((pages.shape[0], 128, 128), dtype=torch.bfloat16, device=dev)
    _check(_lib.fp8_pages_dequant_bf16(_ptr(pages), _ptr(out), pages.shape[0], _stream(dev)))
    return out


# --- workspaces --------------------------------------------------------------------


class Workspace:
    """A zero-filled device buffer that the step calls reuse.

    It starts zero-filled; every successful call leaves its counters and
    histograms zero again, so one buffer serves any number of calls made one
    after another.  Calls that share a workspace must not run concurrently.
    """

    def __init__(self, device, nbytes=0):
        self.device = torch.device(device)
        self.buf = None
        self.ensure(nbytes)

    def ensure(self, nbytes):
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
            assert self.buf.data_ptr() % 256 == 0
        return self.buf

    @property
    def nbytes(self):
        return self.buf.numel()

    def error_word(self):
        """The workspace's device error word as a one-element int32 device
        tensor (a view, no copy): the MONO_DEVERR_* bits the calls on this
        workspace raised.  It can be read after any later synchronisation
        (or copied out asynchronously); check_device_errors() reads and
        clears it."""
        return self.buf[:4].view(torch.int32)


_default_ws = {}


def _workspace(ws, device, nbytes, key):
    if ws is None:
        ws = _default_ws.get((device, key))
        if ws is None:
            ws = _default_ws[(device, key)] = Workspace(device, nbytes)
    ws.ensure(nbytes)
    return ws


def check_device_errors(ws):
    """Synchronise and return (then clear) the device error bits of a workspace."""
    load_library()
    rc = _lib.mono_check_device_errors(_ptr(ws.buf), _stream(ws.device))
    if rc < 0:
        _check(rc)
    return rc


def default_workspaces(device=None):
    """The per-device workspaces used when a call is not given one."""
    dev = torch.device(device) if device is not None else None
    return [w for (d, _), w in _default_ws.items() if dev is None or d == dev]


# --- step tables -------------------------------------------------------------------


def _check_tables(block_table, seq_lens, n_tokens, T):
    _need(T >= 1, f"T must be >= 1, got {T}")
    _need(n_tokens >= 1 and n_tokens % T == 0, f"{n_tokens} tokens for {T} per request")
    B = n_tokens // T
    _need(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32, "tables not int32")
    _need(block_table.dim() == 2 and seq_lens.dim() == 1, "block_table must be 2-D and seq_lens 1-D")
    _need(block_table.shape[0] >= B and seq_lens.shape[0] >= B, "tables shorter than the batch")
    _need(block_table.stride(1) == 1 and block_table.stride(0) == block_table.shape[1], "block table not row-contiguous")
    _need(seq_lens.stride(0) == 1, "seq_lens must be contiguous")
    return B


def index_score_topk_workspace_bytes(B, T, bt_stride, k):
    return int(load_library().mono_index_score_topk_workspace(B, T, bt_stride, k))


def pa_decode_workspace_bytes(B, T, kv_heads, bt_stride, k, sparse):
    return int(load_library().mono_pa_decode_workspace(B, T, kv_heads, bt_stride, k, int(bool(sparse))))


def mono_index_score_topk(index_q, index_pages, block_table, seq_lens, k, *, T=1, out=None,
                          out_scores=None, return_scores=False, workspace=None, page_window=None):
    """Top-k token positions per query token by fp32 index score.

    index_q: bf16 ``[B*T, 128]``; index_pages: uint8 ``[P, 8704]``;
    block_table: int32 ``[>=B, W]`` row-contiguous; seq_lens: int32 ``[>=B]``.
    Returns int32 ``[B*T, k]`` (any order within a row, -1 padding), and the
    fp32 scores of the selected tokens too if ``return_scores``.
    ``page_window=(lo, hi)`` restricts the tokens to block-table columns
    ``[lo, hi)`` (one shard of the indexer's context parallelism).
    """
    return _index_topk("mxfp4", index_q, index_pages, block_table, seq_lens, k, T, out, out_scores, return_scores,
                       workspace, page_window)


def mono_index_score_topk_fp8(index_q, index_pages, block_table, seq_lens, k, *, T=1, out=None,
                              out_scores=None, return_scores=False, workspace=None):
    """:func:`mono_index_score_topk` over an fp8 (e4m3) index pool ``[P, 16384]``."""
    return _index_topk("fp8", index_q, index_pages, block_table, seq_lens, k, T, out, out_scores, return_scores,
                       workspace)


def _index_topk(fmt, index_q, index_pages, block_table, seq_lens, k, T, out, out_scores, return_scores, workspace,
                page_window=None):
    lib = load_library()
    page_bytes, fn = (PAGE_BYTES, lib.mono_index_score_topk) if fmt == "mxfp4" else \
        (FP8_PAGE_BYTES, lib.mono_index_score_topk_fp8)
    _need(index_q.dtype == torch.bfloat16 and index_q.dim() == 2 and index_q.shape[1] == HEAD_DIM,
          "index_q must be bf16 [B*T, 128]")
    _need(index_q.is_contiguous(), "index_q must be contiguous")
    _check_pages(index_pages, "index_pages", 2, page_bytes)
    N = index_q.shape[0]
    B = _check_tables(block_table, seq_lens, N, T)
    dev = _on_gpu(index_q, index_pages, block_table, seq_lens)
    k = int(k)
    _need(k >= 1, "k must be >= 1")
    bt_stride = block_table.shape[1]
    if out is None:
        out = torch.empty((N, k), dtype=torch.int32, device=dev)
    _need(out.dtype == torch.int32 and tuple(out.shape) == (N, k) and out.is_contiguous(), "out must be int32 [B*T, k]")
    if return_scores and out_scores is None:
        out_scores = torch.empty((N, k), dtype=torch.float32, device=dev)
    if out_scores is not None:
        _need(out_scores.dtype == torch.float32 and tuple(out_scores.shape) == (N, k) and out_scores.is_contiguous(),
              "out_scores must be fp32 [B*T, k]")
    nbytes = lib.mono_index_score_topk_workspace(B, T, bt_stride, k)
    _need(nbytes > 0, "invalid shape for mono_index_score_topk")
    ws = _workspace(workspace, dev, nbytes, "topk")
    if page_window is None:
        _check(fn(
            _ptr(index_q), _ptr(index_pages), index_pages.shape[0], _ptr(block_table), bt_stride,
            _ptr(seq_lens), B, T, k, _ptr(out), _ptr(out_scores), _ptr(ws.buf), ws.nbytes, _stream(dev)))
    else:
        _need(fmt == "mxfp4", "page windows are for MXFP4 index pools")
        lo, hi = (int(x) for x in page_window)
        _check(lib.mono_index_score_topk_window(
            _ptr(index_q), _ptr(index_pages), index_pages.shape[0], _ptr(block_table), bt_stride,
            _ptr(seq_lens), B, T, k, lo, hi, _ptr(out), _ptr(out_scores), _ptr(ws.buf), ws.nbytes, _stream(dev)))
    return (out, out_scores) if return_scores else out


def mono_topk_merge(cand_idx, cand_scores, k, *, out=None, out_scores=None):
    """Merge G top-k lists per query token: int32/fp32 ``[G, N, k_in]`` -> (int32 ``[N, k]``, fp32 ``[N, k]``).

    Each row holds the best min(k, candidates) by the index call's rule
    (higher score, ties to the lower position, NaN last) in any order, then
    -1 / NaN padding.
    """
    lib = load_library()
    _need(cand_idx.dtype == torch.int32 and cand_scores.dtype == torch.float32, "candidates must be int32 / fp32")
    _need(cand_idx.dim() == 3 and cand_idx.shape == cand_scores.shape, "candidates must be [G, N, k_in], alike")
    _need(cand_idx.is_contiguous() and cand_scores.is_contiguous(), "candidates must be contiguous")
    G, N, k_in = cand_idx.shape
    dev = _on_gpu(cand_idx, cand_scores)
    k = int(k)
    if out is None:
        out = torch.empty((N, k), dtype=torch.int32, device=dev)
    if out_scores is None:
        out_scores = torch.empty((N, k), dtype=torch.float32, device=dev)
    _need(tuple(out.shape) == (N, k) and out.dtype == torch.int32 and out.is_contiguous(), "out must be int32 [N, k]")
    _need(tuple(out_scores.shape) == (N, k) and out_scores.dtype == torch.float32 and out_scores.is_contiguous(),
          "out_scores must be fp32 [N, k]")
    _check(lib.mono_topk_merge(_ptr(cand_idx), _ptr(cand_scores), G, N, k_in, k, _ptr(out), _ptr(out_scores),
                               _stream(dev)))
    return out, out_scores


def cp_shard_windows(bt_width, shards):
    """Page windows ``[(lo, hi), ...]``: shard r owns columns [r*c, min(W, (r+1)*c)), c = ceil(W / shards)."""
    c = -(-int(bt_width) // int(shards))
    return [(min(r * c, bt_width), min((r + 1) * c, bt_width)) for r in range(shards)]


def indexer_cp_topk(index_q_heads, index_pages, block_table, seq_lens, k, *, T=1, shards=None, workspace=None):
    """Indexer context parallelism on one GPU (``mono_indexer_cp_topk``).

    index_q_heads: bf16 ``[H, B*T, 128]`` (every rank's index-q head).  Shard
    r scores block-table columns ``cp_shard_windows(W, G)[r]`` of every
    request for all H heads in one launch (one read of its window), emitting
    per head its top-k (position, score) pairs; the merge keeps each head's
    top-k over the G lists.  ``shards`` defaults to H.
    Returns int32 ``[H, B*T, k]`` (any order within a row, -1 padding).
    """
    lib = load_library()
    _need(index_q_heads.dim() == 3 and index_q_heads.shape[2] == HEAD_DIM and index_q_heads.dtype == torch.bfloat16,
          "index_q_heads must be bf16 [H, B*T, 128]")
    _need(index_q_heads.is_contiguous(), "index_q_heads must be contiguous")
    H, N = index_q_heads.shape[0], index_q_heads.shape[1]
    G = H if shards is None else int(shards)
    B = _check_tables(block_table, seq_lens, N, T)
    dev = _on_gpu(index_q_heads, index_pages, block_table, seq_lens)
    _check_pages(index_pages, "index_pages", 2, PAGE_BYTES)
    W = block_table.shape[1]
    k = int(k)
    need = int(lib.mono_indexer_cp_topk_workspace(B, T, H, W, k, G))
    _need(need > 0, f"no workspace for B={B} T={T} heads={H} bt_stride={W} k={k} shards={G}")
    ws = _workspace(workspace, dev, need, "cp")
    out = torch.empty((H, N, k), dtype=torch.int32, device=dev)
    _check(lib.mono_indexer_cp_topk(_ptr(index_q_heads), _ptr(index_pages), index_pages.shape[0], _ptr(block_table),
                                    W, _ptr(seq_lens), B, T, H, k, G, _ptr(out), _ptr(ws.buf), ws.nbytes,
                                    _stream(dev)))
    return out


def mono_pa_decode_mxfp4(q, k_pages, v_pages, block_table, seq_lens, selected_idx=None,
                         scale=1.0 / math.sqrt(HEAD_DIM), *, T=1, out=None, workspace=None):
    """Paged GQA decode attention over MXFP4 K/V pages.

    q: bf16 ``[B*T, 16*H, 128]``; k_pages/v_pages: uint8 ``[P, H, 8704]``;
    selected_idx: None (dense: every token up to each query's position) or
    int32 ``[B*T, k]`` (entries < 0 or past the position are skipped).
    Returns bf16 ``[B*T, 16*H, 128]``.
    """
    return _pa_decode("mxfp4", q, k_pages, v_pages, block_table, seq_lens, selected_idx, scale, 1.0, 1.0, T, out,
                      workspace)


def mono_pa_decode_fp8(q, k_pages, v_pages, block_table, seq_lens, selected_idx=None,
                       scale=1.0 / math.sqrt(HEAD_DIM), k_scale=1.0, v_scale=1.0, *, T=1, out=None, workspace=None):
    """:func:`mono_pa_decode_mxfp4` over fp8 (e4m3) K/V pools ``[P, H, 16384]``.

    K values are e4m3 * ``k_scale`` and V values e4m3 * ``v_scale``.
    """
    return _pa_decode("fp8", q, k_pages, v_pages, block_table, seq_lens, selected_idx, scale, k_scale, v_scale, T,
                      out, workspace)


def _pa_decode(fmt, q, k_pages, v_pages, block_table, seq_lens, selected_idx, scale, k_scale, v_scale, T, out,
               workspace):
    lib = load_library()
    page_bytes = PAGE_BYTES if fmt == "mxfp4" else FP8_PAGE_BYTES
    _need(q.dtype == torch.bfloat16 and q.dim() == 3 and q.shape[2] == HEAD_DIM, "q must be bf16 [B*T, 16*H, 128]")
    _need(q.is_contiguous(), "q must be contiguous")
    _check_pages(k_pages, "k_pages", 3, page_bytes)
    _check_pages(v_pages, "v_pages", 3, page_bytes)
    _need(k_pages.shape == v_pages.shape, "k_pages and v_pages must have the same shape")
    H = k_pages.shape[1]
    _need(q.shape[1] == Q_HEADS_PER_KV * H, f"q has {q.shape[1]} heads; the pools have {H} KV heads x 16")
    N = q.shape[0]
    B = _check_tables(block_table, seq_lens, N, T)
    dev = _on_gpu(q, k_pages, v_pages, block_table, seq_lens)
    bt_stride = block_table.shape[1]
    k = 0
    if selected_idx is not None:
        _on_gpu(q, selected_idx)
        _need(selected_idx.dtype == torch.int32 and selected_idx.dim() == 2 and selected_idx.shape[0] == N
              and selected_idx.is_contiguous(), "selected_idx must be int32 [B*T, k], contiguous")
        k = selected_idx.shape[1]
        _need(k >= 1, "selected_idx must have k >= 1 columns")
    if out is None:
        out = torch.empty_like(q)
    _need(out.dtype == torch.bfloat16 and out.shape == q.shape and out.is_contiguous(), "out must match q")
    nbytes = lib.mono_pa_decode_workspace(B, T, H, bt_stride, k, int(selected_idx is not None))
    _need(nbytes > 0, "invalid shape for mono_pa_decode_mxfp4")
    ws = _workspace(workspace, dev, nbytes, "pa")
    args = [_ptr(q), _ptr(k_pages), _ptr(v_pages), k_pages.shape[0], H, _ptr(block_table), bt_stride,
            _ptr(seq_lens), B, T, _ptr(selected_idx), k, ctypes.c_float(float(scale))]
    if fmt == "mxfp4":
        _check(lib.mono_pa_decode_mxfp4(*args, _ptr(out), _ptr(ws.buf), ws.nbytes, _stream(dev)))
    else:
        _check(lib.mono_pa_decode_fp8(*args, ctypes.c_float(float(k_scale)), ctypes.c_float(float(v_scale)),
                                      _ptr(out), _ptr(ws.buf), ws.nbytes, _stream(dev)))
    return out


def sparse_decode_workspace_bytes(B, T, kv_heads, bt_stride, k):
    return int(load_library().mono_sparse_decode_workspace(B, T, kv_heads, bt_stride, k))


def mono_sparse_decode_mxfp4(index_q, index_pages, q, k_pages, v_pages, block_table, seq_lens, k,
                             scale=1.0 / math.sqrt(HEAD_DIM), *, T=1, out=None, selected_idx=None,
                             workspace=None):
    """One sparse decode step in one launch: index top-k, then attention over the selection.

    Arguments as for :func:`mono_index_score_topk` and :func:`mono_pa_decode_mxfp4`.
    Returns ``(out, selected_idx)``: bf16 ``[B*T, 16*H, 128]`` and int32 ``[B*T, k]``.
    """
    return _sparse_decode("mxfp4", index_q, index_pages, q, k_pages, v_pages, block_table, seq_lens, k, scale, 1.0,
                          1.0, T, out, selected_idx, workspace)


def mono_sparse_decode_fp8(index_q, index_pages, q, k_pages, v_pages, block_table, seq_lens, k,
                           scale=1.0 / math.sqrt(HEAD_DIM), k_scale=1.0, v_scale=1.0, *, T=1, out=None,
                           selected_idx=None, workspace=None):
    """:func:`mono_sparse_decode_mxfp4` over fp8 (e4m3) pools: index ``[P, 16384]``, K/V ``[P, H, 16384]``."""
    return _sparse_decode("fp8", index_q, index_pages, q, k_pages, v_pages, block_table, seq_lens, k, scale, k_scale,
                          v_scale, T, out, selected_idx, workspace)


def _sparse_decode(fmt, index_q, index_pages, q, k_pages, v_pages, block_table, seq_lens, k, scale, k_scale, v_scale,
                   T, out, selected_idx, workspace):
    lib = load_library()
    page_bytes = PAGE_BYTES if fmt == "mxfp4" else FP8_PAGE_BYTES
    _need(index_q.dtype == torch.bfloat16 and index_q.dim() == 2 and index_q.shape[1] == HEAD_DIM,
          "index_q must be bf16 [B*T, 128]")
    _need(index_q.is_contiguous(), "index_q must be contiguous")
    _check_pages(index_pages, "index_pages", 2, page_bytes)
    _need(q.dtype == torch.bfloat16 and q.dim() == 3 and q.shape[2] == HEAD_DIM, "q must be bf16 [B*T, 16*H, 128]")
    _need(q.is_contiguous(), "q must be contiguous")
    _check_pages(k_pages, "k_pages", 3, page_bytes)
    _check_pages(v_pages, "v_pages", 3, page_bytes)
    _need(k_pages.shape == v_pages.shape, "k_pages and v_pages must have the same shape")
    _need(index_pages.shape[0] == k_pages.shape[0], "the index pool and the K/V pools must have the same page count")
    H = k_pages.shape[1]
    _need(q.shape[1] == Q_HEADS_PER_KV * H, f"q has {q.shape[1]} heads; the pools have {H} KV heads x 16")
    N = q.shape[0]
    _need(index_q.shape[0] == N, "index_q and q must have the same number of query tokens")
    B = _check_tables(block_table, seq_lens, N, T)
    dev = _on_gpu(index_q, index_pages, q, k_pages, v_pages, block_table, seq_lens)
    k = int(k)
    _need(k >= 1, "k must be >= 1")
    bt_stride = block_table.shape[1]
    if selected_idx is None:
        selected_idx = torch.empty((N, k), dtype=torch.int32, device=dev)
    _on_gpu(q, selected_idx)
    _need(selected_idx.dtype == torch.int32 and tuple(selected_idx.shape) == (N, k) and selected_idx.is_contiguous(),
          "selected_idx must be int32 [B*T, k]")
    if out is None:
        out = torch.empty_like(q)
    _need(out.dtype == torch.bfloat16 and out.shape == q.shape and out.is_contiguous(), "out must match q")
    nbytes = lib.mono_sparse_decode_workspace(B, T, H, bt_stride, k)
    _need(nbytes > 0, "invalid shape for mono_sparse_decode_mxfp4")
    ws = _workspace(workspace, dev, nbytes, "step")
    args = [_ptr(index_q), _ptr(index_pages), _ptr(q), _ptr(k_pages), _ptr(v_pages), k_pages.shape[0], H,
            _ptr(block_table), bt_stride, _ptr(seq_lens), B, T, k, ctypes.c_float(float(scale))]
    tail = [_ptr(selected_idx), _ptr(out), _ptr(ws.buf), ws.nbytes, _stream(dev)]
    if fmt == "mxfp4":
        _check(lib.mono_sparse_decode_mxfp4(*args, *tail))
    else:
        _check(lib.mono_sparse_decode_fp8(*args, ctypes.c_float(float(k_scale)), ctypes.c_float(float(v_scale)),
                                          *tail))
    return out, selected_idx


NOALLOC_SCRATCH_BYTES = 64 << 20


def mono_sparse_decode_mxfp4_noalloc(index_q, index_pages, q, k_pages, v_pages, block_table, seq_lens, k, scale,
                                     out, selected_idx, *, T=1, err=None):
    """:func:`mono_sparse_decode_mxfp4` without a workspace and without any allocation.

    The library's static per-device scratch (64 MiB) serves as the
    workspace; ``out`` and ``selected_idx`` must be given.  ``err``: None or
    an int32/uint32 device tensor of one element into which the call's
    device error bits are OR-ed.  Calls that overlap in time on one device
    race.  Returns ``(out, selected_idx)``.
    """
    lib = load_library()
    _need(index_q.dtype == torch.bfloat16 and index_q.dim() == 2 and index_q.shape[1] == HEAD_DIM,
          "index_q must be bf16 [B*T, 128]")
    _need(index_q.is_contiguous(), "index_q must be contiguous")
    _check_pages(index_pages, "index_pages", 2)
    _need(q.dtype == torch.bfloat16 and q.dim() == 3 and q.shape[2] == HEAD_DIM, "q must be bf16 [B*T, 16*H, 128]")
    _need(q.is_contiguous(), "q must be contiguous")
    _check_pages(k_pages, "k_pages", 3)
    _check_pages(v_pages, "v_pages", 3)
    _need(k_pages.shape == v_pages.shape, "k_pages and v_pages must have the same shape")
    _need(index_pages.shape[0] == k_pages.shape[0], "the index pool and the K/V pools must have the same page count")
    H = k_pages.shape[1]
    _need(q.shape[1] == Q_HEADS_PER_KV * H, f"q has {q.shape[1]} heads; the pools have {H} KV heads x 16")
    N = q.shape[0]
    _need(index_q.shape[0] == N, "index_q and q must have the same number of query tokens")
    B = _check_tables(block_table, seq_lens, N, T)
    dev = _on_gpu(index_q, index_pages, q, k_pages, v_pages, block_table, seq_lens, out, selected_idx)
    k = int(k)
    _need(k >= 1, "k must be >= 1")
    _need(selected_idx.dtype == torch.int32 and tuple(selected_idx.shape) == (N, k) and selected_idx.is_contiguous(),
          "selected_idx must be int32 [B*T, k]")
    _need(out.dtype == torch.bfloat16 and out.shape == q.shape and out.is_contiguous(), "out must match q")
    if err is not None:
        _on_gpu(q, err)
        _need(err.dtype in (torch.int32, torch.uint32) and err.numel() == 1, "err must be one 32-bit device word")
    _check(lib.mono_sparse_decode_mxfp4_noalloc(
        _ptr(index_q), _ptr(index_pages), _ptr(q), _ptr(k_pages), _ptr(v_pages), k_pages.shape[0], H,
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B, T, k, ctypes.c_float(float(scale)),
        _ptr(selected_idx), _ptr(out), _ptr(err), _stream(dev)))
    return out, selected_idx


def mono_insert_mxfp4(slots, *, k_rows=None, v_rows=None, index_rows=None, k_pages=None, v_pages=None,
                      index_pages=None, workspace=None):
    """Quantise bf16 rows to MXFP4 and write them into the pages through ``slots``.

    ``slots``: int64 ``[n]``, slot s = row s % 128 of page s // 128; negative
    slots are skipped.  ``k_rows``/``v_rows``: bf16 ``[n, H, 128]`` into
    ``k_pages``/``v_pages`` ``[pages, H, 8704]``; ``index_rows``: bf16
    ``[n, 128]`` into ``index_pages`` ``[pages, 8704]``.  Any cache may be
    left out (rows and pages both None).  A slot past the pools sets
    ``DEVERR_SLOT`` in the workspace's error word; the workspace used is
    returned, for :func:`check_device_errors`.
    """
    lib = load_library()
    _need(slots.dtype == torch.int64 and slots.dim() == 1 and slots.is_contiguous(), "slots must be int64 [n]")
    n = slots.shape[0]
    pairs = ((k_rows, k_pages, "k", 3), (v_rows, v_pages, "v", 3), (index_rows, index_pages, "index", 2))
    given = [(r, p) for r, p, _, _ in pairs if r is not None or p is not None]
    _need(len(given) > 0, "no cache to write")
    H = 0
    num_pages = None
    for rows, pages, name, ndim in pairs:
        if rows is None and pages is None:
            continue
        _need(rows is not None and pages is not None, f"{name}_rows and {name}_pages go together")
        _check_pages(pages, f"{name}_pages", ndim)
        _need(rows.dtype == torch.bfloat16 and rows.is_contiguous(), f"{name}_rows must be contiguous bf16")
        heads = pages.shape[1] if ndim == 3 else 1
        want = (n, heads, HEAD_DIM) if ndim == 3 else (n, HEAD_DIM)
        _need(tuple(rows.shape) == want, f"{name}_rows must be {want}, got {tuple(rows.shape)}")
        if ndim == 3:
            _need(H in (0, heads), "k_pages and v_pages must have the same number of heads")
            H = heads
        _need(num_pages in (None, pages.shape[0]), "every pool must have the same page count")
        num_pages = pages.shape[0]
    dev = _on_gpu(slots, *[t for pair in given for t in pair])
    ws = _workspace(workspace, dev, 256, "insert")
    _check(lib.mono_insert_mxfp4(
        _ptr(k_rows), _ptr(v_rows), _ptr(index_rows), _ptr(slots), n, H, _ptr(k_pages), _ptr(v_pages),
        _ptr(index_pages), num_pages, _ptr(ws.buf), _stream(dev)))
    return ws


def bench_read(pages, page_ids=None, grid=512, sink=None):
    """Read-bandwidth reference: stream every byte of ``pages`` ``[n, 8704]``
    (``page_ids`` None) or gather the pages ``page_ids`` (int32 ``[m]``) with
    the index scan's lane pattern.  Returns the sink (one word per workgroup)."""
    lib = load_library()
    _check_pages(pages, "pages", 2)
    dev = _on_gpu(pages)
    mode = 0 if page_ids is None else 1
    n = pages.shape[0]
    if mode == 1:
        _on_gpu(pages, page_ids)
        _need(page_ids.dtype == torch.int32 and page_ids.dim() == 1 and page_ids.is_contiguous(),
              "page_ids must be int32 [m], contiguous")
        n = page_ids.shape[0]
    if sink is None:
        sink = torch.empty(grid, dtype=torch.int32, device=dev)
    _need(sink.dtype == torch.int32 and sink.numel() >= grid, "sink must hold grid int32 words")
    _check(lib.mono_bench_read(_ptr(pages), _ptr(page_ids), n, mode, int(grid), _ptr(sink), _stream(dev)))
    return sink


def bench_scan(index_q, index_pages, block_table, seq_lens, chunk_pages, variant, hist=None, err=None):
    """The index scan phase on the matrix cores (variant 0) or the VALU
    (variant 1): bf16 ``index_q [B, 128]``, one query token per request.
    Adds each request's score histogram (2048 bins) to ``hist`` (int32
    ``[B, 2048]``, zeroed when created here); returns (hist, err word)."""
    lib = load_library()
    _need(index_q.dtype == torch.bfloat16 and index_q.dim() == 2 and index_q.shape[1] == HEAD_DIM
          and index_q.is_contiguous(), "index_q must be bf16 [B, 128], contiguous")
    _check_pages(index_pages, "index_pages", 2, PAGE_BYTES)
    B = index_q.shape[0]
    B = _check_tables(block_table, seq_lens, B, 1)
    dev = _on_gpu(index_q, index_pages, block_table, seq_lens)
    if hist is None:
        hist = torch.zeros((B, 2048), dtype=torch.int32, device=dev)
    if err is None:
        err = torch.zeros(1, dtype=torch.int32, device=dev)
    _need(hist.dtype == torch.int32 and hist.is_contiguous() and hist.numel() >= B * 2048, "hist must be int32 [B, 2048]")
    _check(lib.mono_bench_scan(_ptr(index_q), _ptr(index_pages), index_pages.shape[0], _ptr(block_table),
                               block_table.shape[1], _ptr(seq_lens), B, int(chunk_pages), int(variant), _ptr(hist),
                               _ptr(err), _stream(dev)))
    return hist, err


# --- per-kernel timing ---------------------------------------------------------------


class KernelTimer:
    """Times every kernel the library launches with HIP events (context manager).

    ``with KernelTimer() as kt: ...`` then ``kt.mean_us`` maps kernel name to
    mean microseconds per launch and ``kt.launches`` to launch counts.
    """

    def __init__(self, capacity=4096):
        self.capacity = capacity
        self.mean_us = {}
        self.launches = {}

    def __enter__(self):
        _check(load_library().mono_profile_start(self.capacity))
        return self

    def __exit__(self, *exc):
        n = 64  # more than the library's kernel ids (mono_profile_stop returns how many it has)
        tot = (ctypes.c_double * n)()
        cnt = (ctypes.c_int * n)()
        rc = _lib.mono_profile_stop(tot, cnt, n)
        if rc < 0:
            _check(rc)
        for k in range(min(rc, n)):
            if cnt[k]:
                name = _lib.mono_kernel_name(k).decode()
                self.launches[name] = cnt[k]
                self.mean_us[name] = tot[k] * 1000.0 / cnt[k]
        return False
