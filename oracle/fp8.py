"""fp8 (e4m3) cache pages and their exact values (CPU oracle, test infrastructure).

Source: page *vllm.models.minimax_m3.amd.mono.weights*, ``SparseMoeLayer``
(the index cache is ``[blocks, block, head_dim]`` fp8 with shared block
ids; the layer's attention object carries the KV cache views and their
scales) and page *vllm.models.minimax_m3.amd.mono.dispatch*,
``_config_refusal`` (that build requires a KV cache dtype starting with
"fp8" and an fp8 index cache).  This is the older build's cache format; the
MXFP4 pages replace it in the later build.

Readings, where the pages only say "fp8":

* The element format is OCP FP8 E4M3 ("e4m3fn", the one gfx950 converts
  natively): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
  exponent 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN;
  there are no infinities, so the largest value is 448.
* A page holds 128 tokens x 128 elements, one byte each, row-major:
  element i of row r is byte 128*r + i, 16384 bytes per page.  K and V
  pools are ``[pages, kv_heads, 16384]``, the index pool ``[pages, 16384]``.
* K and V carry one fp32 scale each for the whole tensor (the "scales" the
  layer's attention object holds): the value of a K element is
  e4m3(code) * k_scale, of a V element e4m3(code) * v_scale.  The index
  cache has no scale: its values are the e4m3 values themselves.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use this module.
"""

import numpy as np

PAGE_TOKENS = 128
ROW_ELEMS = 128
PAGE_BYTES = PAGE_TOKENS * ROW_ELEMS  # 16384


def e4m3_value(code):
    """float64 value of e4m3 code(s) 0..255 from the bit fields; NaN for 0x7F / 0xFF."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where((code & 0x80) != 0, -1.0, 1.0)
    exp = (code >> 3) & 0xF
    man = code & 0x7
    normal = np.ldexp(1.0 + man / 8.0, exp - 7)
    subnormal = np.ldexp(man / 8.0, -6)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return sign * mag


def rows_view(pages):
    """``[..., 128, 128]`` uint8 view of fp8 pages ``[..., 16384]`` (row r, element i = byte 128r + i)."""
    pages = np.asarray(pages)
    if pages.dtype != np.uint8 or pages.ndim < 1 or pages.shape[-1] != PAGE_BYTES:
        raise ValueError(f"fp8 pages must be uint8 [..., {PAGE_BYTES}], got {pages.dtype} {pages.shape}")
    return pages.reshape(*pages.shape[:-1], PAGE_TOKENS, ROW_ELEMS)


def dequant(pages):
    """Exact float64 values ``[..., 128, 128]`` of fp8 pages ``[..., 16384]`` (no tensor scale)."""
    return e4m3_value(rows_view(pages))
