"""MXFP4 page geometry, exact dequantisation and the cache insert (CPU oracle,
test infrastructure).

Source: page *vllm.models.minimax_m3.amd.ops.mxfp4_pages*, module docstring
and the function ``mxfp4_page_views``.  One 128-token page of one head holds
the 128 rows of 128-wide e2m1 data, two elements per byte with the even
element in the low nibble (64 B per row), and then one e8m0 scale byte per
32 elements (4 B per row).  The page is 128 x 64 + 128 x 4 = 8704 B and has
no global scale.  K, V and the single index-key head all use this page.

The numeric meaning of the two element formats is the OCP Microscaling one,
which the page names but does not spell out:

* e2m1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa, so the
  magnitudes of codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Code 8 is -0.0.
* e8m0: the byte e means 2**(e - 127); 0xFF is NaN.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use this module.
"""

import numpy as np

PAGE_TOKENS = 128  # rows (tokens) per page
ROW_ELEMS = 128  # elements per row (head_dim)
SCALE_BLOCK = 32  # elements sharing one e8m0 scale
DATA_BYTES = ROW_ELEMS // 2  # 64: two e2m1 elements per byte
SCALE_BYTES = ROW_ELEMS // SCALE_BLOCK  # 4
DATA_REGION = PAGE_TOKENS * DATA_BYTES  # 8192: the scale region starts here
PAGE_BYTES = DATA_REGION + PAGE_TOKENS * SCALE_BYTES  # 8704

# e2m1 magnitudes of codes 0..7 (OCP MX FP4); codes 8..15 are their negatives.
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def page_views(pages):
    """(data, scale) zero-copy views of uint8 pages ``[..., 8704]``.

    The page geometry of the mxfp4_pages page (module docstring and
    ``mxfp4_page_views``): bytes 0..8191 of a page are its 128 rows of 64
    packed e2m1 bytes, bytes 8192..8703 its 128 rows of 4 e8m0 bytes.  The
    data view is the first region of the last axis split into
    ``[..., 128, 64]``, the scale view the second split into ``[..., 128, 4]``;
    both keep the leading dims and their strides, and writes through them
    land in ``pages``.  A dtype other than uint8, a last dim other than 8704
    or bytes of a page that are not adjacent raise ValueError.
    """
    pages = np.asarray(pages)
    if pages.dtype != np.uint8:
        raise ValueError(f"page views need uint8 bytes, not {pages.dtype}")
    if pages.ndim < 1 or pages.shape[-1] != PAGE_BYTES:
        raise ValueError(f"the last axis must be one {PAGE_BYTES}-byte page; shape is {pages.shape}")
    if pages.strides[-1] != 1:
        raise ValueError(f"the bytes of a page must be adjacent (last-axis stride {pages.strides[-1]}, not 1)")
    lead = pages.shape[:-1]
    data = pages[..., :DATA_REGION].view()
    data.shape = (*lead, PAGE_TOKENS, DATA_BYTES)  # splits the unit-stride axis in place: never a copy
    scale = pages[..., DATA_REGION:].view()
    scale.shape = (*lead, PAGE_TOKENS, SCALE_BYTES)
    return data, scale


def pack(codes, scales):
    """Pages ``[..., 8704]`` from one e2m1 code per byte and the e8m0 scales.

    ``codes``: uint8 ``[..., 128, 128]`` (only the low 4 bits are used);
    ``scales``: uint8 ``[..., 128, 4]``.  Element 2c of a row goes to the low
    nibble of data byte c and element 2c+1 to its high nibble (mxfp4_pages
    page, module docstring: "the low nibble the even one").
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lead = codes.shape[:-2]
    assert codes.shape[-2:] == (PAGE_TOKENS, ROW_ELEMS)
    assert scales.shape == (*lead, PAGE_TOKENS, SCALE_BYTES)
    even = codes[..., 0::2] & 0x0F
    odd = codes[..., 1::2] & 0x0F
    data = (even | (odd << 4)).astype(np.uint8)  # [..., 128, 64]
    pages = np.empty((*lead, PAGE_BYTES), dtype=np.uint8)
    pages[..., :DATA_REGION] = data.reshape(*lead, DATA_REGION)
    pages[..., DATA_REGION:] = scales.reshape(*lead, PAGE_TOKENS * SCALE_BYTES)
    return pages


def unpack(pages):
    """Inverse of ``pack``: (codes ``[..., 128, 128]``, scales ``[..., 128, 4]``)."""
    data, scale = page_views(pages)
    lead = data.shape[:-2]
    codes = np.empty((*lead, PAGE_TOKENS, ROW_ELEMS), dtype=np.uint8)
    codes[..., 0::2] = data & 0x0F
    codes[..., 1::2] = data >> 4
    return codes, np.array(scale, dtype=np.uint8)


def _e2m1_table():
    """float64 values of the 16 e2m1 codes: bits 2..0 give the magnitude and
    bit 3 the sign (code 8 is -0.0)."""
    mags = np.asarray(E2M1_MAGNITUDES, dtype=np.float64)
    return np.concatenate([mags, -mags])


_E2M1_TABLE = _e2m1_table()


def e2m1_value(code):
    """float64 value of e2m1 code(s) 0..15; code 8 gives -0.0."""
    code = np.asarray(code)
    return _E2M1_TABLE[(code & 15).astype(np.uint8)]


def e8m0_value(e):
    """float64 value 2**(e - 127) of e8m0 byte(s); 255 gives NaN."""
    e = np.asarray(e, dtype=np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))


def dequant(pages):
    """Exact float64 values ``[..., 128, 128]`` of MXFP4 pages ``[..., 8704]``.

    Element i of row r is e2m1(code[r, i]) * 2**(e[r, i // 32] - 127): the
    32-element blocks of a row are contiguous and each has its own scale
    byte (mxfp4_pages page, module docstring: one e8m0 scale per 32
    elements).  Every product is exact in float64.
    """
    codes, scales = unpack(pages)
    block_scale = e8m0_value(scales)  # [..., 128, 4]: block g of row r
    values = e2m1_value(codes).reshape(*codes.shape[:-1], SCALE_BYTES, SCALE_BLOCK)  # [..., 128, 4, 32]
    return (values * block_scale[..., None]).reshape(codes.shape)


def round_to_f32(x):
    """float64 -> float32 with round-to-nearest-even (numpy's cast)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_to_bf16_bits(x):
    """float64 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    Goes float64 -> float32 (RNE) -> bfloat16 (RNE on the top 16 bits).  For
    values with at most 8 significant bits, such as every finite MXFP4 value,
    both roundings are exact, so the result is the value itself.
    """
    f = round_to_f32(x)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = np.where(nan, (u >> 16) | 0x40, rounded)
    return out.astype(np.uint16)


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Writing rows into pages (the cache insert).
#
# The dispatch page (vllm.models.minimax_m3.amd.mono.dispatch, _slots_shared
# and _step_refusal) says the kernels insert K/V and the index key through
# one int64 page-128 slot mapping shared by both caches; the mxfp4_pages page
# names the writer but prints no rule for choosing the scale or rounding.
# The reading taken is the OCP Microscaling Formats v1.0 conversion for
# MXFP4: per block of 32 elements the shared exponent is
# floor(log2(max |v|)) - 2 (2 = the largest exponent of e2m1), and each
# element v / 2**shared is rounded to the nearest e2m1 value, ties to the
# even code, magnitudes above 6 saturating to 6.  Readings where that
# specification leaves a choice:
#   * an all-zero block gets scale byte 0 and codes 0 (or 8 for -0.0);
#   * a block holding NaN or +-inf gets scale byte 0xFF (NaN) and codes 0;
#   * the scale byte is clamped to 0..254.
# Slot s is row s % 128 of page s // 128; a negative slot is skipped.
# ---------------------------------------------------------------------------
def quantize_block(v):
    """(codes [32] uint8, scale byte) of one 32-element block of float values."""
    v = np.asarray(v, dtype=np.float64)
    assert v.shape == (SCALE_BLOCK,)
    sign = np.signbit(v)
    if not np.all(np.isfinite(v)):
        return np.zeros(SCALE_BLOCK, dtype=np.uint8), 0xFF
    amax = float(np.max(np.abs(v)))
    if amax == 0.0:
        return np.where(sign, 8, 0).astype(np.uint8), 0
    # floor(log2 amax), exactly: frexp gives amax = m * 2**e with m in [0.5, 1).
    shared = (int(np.frexp(amax)[1]) - 1) - 2
    byte = min(max(shared + 127, 0), 254)
    q = np.abs(v) / 2.0 ** (byte - 127)
    codes = np.empty(SCALE_BLOCK, dtype=np.uint8)
    for n, x in enumerate(q):
        codes[n] = _nearest_e2m1(x) | (8 if sign[n] else 0)
    return codes, byte


def _nearest_e2m1(x):
    """Code 0..7 of the e2m1 magnitude nearest x >= 0, ties to the even code, saturating."""
    if x >= E2M1_MAGNITUDES[-1]:
        # Saturation, stated directly: for very large x the float64 distances
        # to 4 and to 6 round to the same number and would tie.
        return 7
    best = None
    for code, mag in enumerate(E2M1_MAGNITUDES):
        d = abs(x - mag)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


def quantize_rows(rows):
    """(codes [..., 128] uint8, scales [..., 4] uint8) of float rows [..., 128]."""
    rows = np.asarray(rows, dtype=np.float64)
    lead = rows.shape[:-1]
    flat = rows.reshape(-1, SCALE_BYTES, SCALE_BLOCK)
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty(flat.shape[:-1], dtype=np.uint8)
    for r in range(flat.shape[0]):
        for b in range(SCALE_BYTES):
            codes[r, b], scales[r, b] = quantize_block(flat[r, b])
    return codes.reshape(*lead, ROW_ELEMS), scales.reshape(*lead, SCALE_BYTES)


def insert_rows(pool, rows, slots):
    """Write float rows [n, heads, 128] into pool [pages, heads, 8704] through slots [n].

    Returns the pool (a copy) and the list of token indices whose slot was
    past the pool (those rows are not written).
    """
    pool = np.array(pool, dtype=np.uint8, copy=True)
    rows = np.asarray(rows, dtype=np.float64)
    n_pages = pool.shape[0]
    codes, scales = quantize_rows(rows)
    data, scale = page_views(pool)
    skipped = []
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        page, row = divmod(int(s), PAGE_TOKENS)
        if page >= n_pages:
            skipped.append(t)
            continue
        for h in range(rows.shape[1]):
            c = codes[t, h]
            data[page, h, row] = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)
            scale[page, h, row] = scales[t, h]
    return pool, skipped
