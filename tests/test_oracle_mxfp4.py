"""Pins of the oracle's MXFP4 geometry, packing and value tables.

Each test checks the oracle against something other than itself: the
geometry the mxfp4_pages page prints, hand-worked fixtures under
``tests/golden/``, the OCP e2m1 bit-field decode, torch's float8_e8m0fnu
conversion, and exhaustive round trips.
"""

import os

import numpy as np
import pytest
import torch

from oracle import mxfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# --- geometry -----------------------------------------------------------------


def test_page_size_closed_form():
    # [128 tokens x 64 B data][128 tokens x 4 B scale] = 8704 B = 128 x 68 B
    assert mxfp4.PAGE_BYTES == 128 * 64 + 128 * 4 == 128 * 68 == 8704
    assert mxfp4.DATA_REGION == 8192
    assert mxfp4.DATA_BYTES == 64 and mxfp4.SCALE_BYTES == 4


def _offset(view, base):
    return view.__array_interface__["data"][0] - base.__array_interface__["data"][0]


def test_page_views_match_golden_geometry():
    g = {r[0]: [int(x) for x in r[1:]] for r in _read_golden("page_views_geometry.txt")}
    buf = np.zeros(5 * 2 * 8704 + 64, dtype=np.uint8)
    pool = buf[g["pool_offset"][0] : g["pool_offset"][0] + 3 * 2 * 8704].reshape(3, 2, 8704)
    assert list(pool.shape) == g["pool_shape"] and list(pool.strides) == g["pool_strides"]
    data, scale = mxfp4.page_views(pool)
    assert list(data.shape) == g["data_shape"]
    assert list(data.strides) == g["data_strides"]
    assert _offset(data, buf) == g["data_offset"][0]
    assert list(scale.shape) == g["scale_shape"]
    assert list(scale.strides) == g["scale_strides"]
    assert _offset(scale, buf) == g["scale_offset"][0]
    # element addresses: mark one byte in the buffer and find it through the views
    buf[g["data_addr_2_1_5_7"][0]] = 0xAB
    buf[g["scale_addr_1_0_127_3"][0]] = 0xCD
    assert data[2, 1, 5, 7] == 0xAB and np.count_nonzero(data == 0xAB) == 1
    assert scale[1, 0, 127, 3] == 0xCD and np.count_nonzero(scale == 0xCD) == 1


def test_page_views_match_torch_as_strided():
    """Same bytes as torch.as_strided views built the way the page describes."""
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 256, size=(4 * 3 * 8704 + 100,), dtype=np.uint8)
    t = torch.from_numpy(raw)
    off = 8704 * 3 + 17  # an odd storage offset
    pool_t = t.as_strided((2, 3, 8704), (3 * 8704, 8704, 1), off)
    lead, ls = (2, 3), (3 * 8704, 8704)
    data_t = t.as_strided((*lead, 128, 64), (*ls, 64, 1), off)
    scale_t = t.as_strided((*lead, 128, 4), (*ls, 4, 1), off + 128 * 64)
    data, scale = mxfp4.page_views(pool_t.numpy())
    np.testing.assert_array_equal(data, data_t.numpy())
    np.testing.assert_array_equal(scale, scale_t.numpy())
    # index-K pool [pages, 8704]
    pool2 = t.as_strided((5, 8704), (8704, 1), 3)
    d2, s2 = mxfp4.page_views(pool2.numpy())
    np.testing.assert_array_equal(d2, t.as_strided((5, 128, 64), (8704, 64, 1), 3).numpy())
    np.testing.assert_array_equal(s2, t.as_strided((5, 128, 4), (8704, 4, 1), 3 + 8192).numpy())


def test_page_views_errors():
    with pytest.raises(ValueError):
        mxfp4.page_views(np.zeros((2, 8704), dtype=np.int8))
    with pytest.raises(ValueError):
        mxfp4.page_views(np.zeros((2, 8703), dtype=np.uint8))
    strided = np.zeros((2, 2 * 8704), dtype=np.uint8)[:, ::2]
    assert strided.shape == (2, 8704)
    with pytest.raises(ValueError):
        mxfp4.page_views(strided)


# --- packing --------------------------------------------------------------------


def test_nibble_packing_golden():
    for even, odd, byte in _read_golden("nibble_packing.txt"):
        codes = np.zeros((128, 128), dtype=np.uint8)
        codes[3, 10] = int(even)
        codes[3, 11] = int(odd)
        page = mxfp4.pack(codes, np.full((128, 4), 127, dtype=np.uint8))
        assert page[3 * 64 + 5] == int(byte, 16), (even, odd, byte)
        back, _ = mxfp4.unpack(page)
        assert back[3, 10] == int(even) and back[3, 11] == int(odd)


def test_pack_unpack_exhaustive_round_trip():
    """All 16 x 16 nibble pairs in every byte position and all 256 scale bytes."""
    n = 16
    codes = np.zeros((n, 128, 128), dtype=np.uint8)
    pairs = np.array([(a, b) for a in range(16) for b in range(16)], dtype=np.uint8)  # 256
    # page p, row r, byte c carries pair (p*128*64 + r*64 + c) mod 256
    idx = (np.arange(n * 128 * 64) % 256).reshape(n, 128, 64)
    codes[..., 0::2] = pairs[idx, 0]
    codes[..., 1::2] = pairs[idx, 1]
    scales = (np.arange(n * 128 * 4) % 256).astype(np.uint8).reshape(n, 128, 4)
    pages = mxfp4.pack(codes, scales)
    assert pages.shape == (n, 8704)
    c2, s2 = mxfp4.unpack(pages)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scales)
    # every byte value occurs in the data region, every scale byte in the scale region
    assert set(np.unique(pages[:, :8192])) == set(range(256))
    assert set(np.unique(pages[:, 8192:])) == set(range(256))
    # upper nibbles of the code input are ignored
    np.testing.assert_array_equal(mxfp4.pack(codes | 0xF0, scales), pages)


# --- value tables ---------------------------------------------------------------


def _ocp_e2m1(code):
    """Decode from the bit fields, independent of the oracle's table."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


def test_e2m1_values():
    golden = {int(c): float(v) for c, v in _read_golden("e2m1_values.txt")}
    vals = mxfp4.e2m1_value(np.arange(16))
    for c in range(16):
        assert vals[c] == golden[c] == _ocp_e2m1(c)
        assert np.signbit(vals[c]) == bool(c & 8)  # code 8 is -0.0
    assert set(np.abs(vals)) == {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    assert np.all(np.diff(vals[:8]) > 0)
    np.testing.assert_array_equal(vals[8:], -vals[:8])


def test_e8m0_values_against_torch():
    e = np.arange(256)
    ours = mxfp4.e8m0_value(e)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    assert ours[127] == 1.0 and ours[0] == 2.0**-127 and np.isnan(ours[255])


# --- dequantisation -------------------------------------------------------------


def test_dequant_single_element_positions():
    """One nonzero element at a time: its value and position come out alone.

    Scales differ per (row, block), so a wrong block (e.g. i % 4 for i // 32),
    a swapped nibble or a wrong row shows up as a wrong value or position.
    """
    scales = np.zeros((128, 4), dtype=np.uint8)
    for r in range(128):
        for g in range(4):
            scales[r, g] = 100 + (r * 4 + g) % 50
    for r, i, code in [(0, 0, 2), (0, 1, 7), (5, 31, 9), (5, 32, 3), (77, 64, 15), (127, 127, 6), (64, 96, 1)]:
        codes = np.zeros((128, 128), dtype=np.uint8)
        codes[r, i] = code
        x = mxfp4.dequant(mxfp4.pack(codes, scales))
        nz = np.argwhere(x != 0)
        assert nz.tolist() == [[r, i]]
        expect = _ocp_e2m1(code) * 2.0 ** (int(scales[r, i // 32]) - 127)
        assert x[r, i] == expect


def test_dequant_against_independent_decode():
    rng = np.random.default_rng(11)
    pages = rng.integers(0, 256, size=(3, 8704), dtype=np.uint8)
    x = mxfp4.dequant(pages)
    # independent decode: bytes -> nibbles by integer division, torch e8m0
    data = pages[:, :8192].reshape(3, 128, 64).astype(np.int64)
    lo, hi = data % 16, data // 16
    sc = torch.from_numpy(pages[:, 8192:].reshape(3, 128, 4).copy()).view(torch.float8_e8m0fnu)
    sc = sc.to(torch.float64).numpy()
    table = np.array([_ocp_e2m1(c) for c in range(16)])
    for p in range(3):
        for r in range(0, 128, 9):
            for i in range(128):
                nib = lo[p, r, i // 2] if i % 2 == 0 else hi[p, r, i // 2]
                want = table[nib] * sc[p, r, i // 32]
                assert x[p, r, i] == want or (np.isnan(want) and np.isnan(x[p, r, i]))


def test_round_to_bf16_bits():
    vals = np.array([1.0, -2.5, 3.0 * 2.0**-130, 6.0 * 2.0**127, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-9])
    bits = mxfp4.round_to_bf16_bits(vals)
    ref = torch.from_numpy(vals).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = mxfp4.bf16_bits_to_f64(bits)
    assert back[0] == 1.0 and back[1] == -2.5 and np.isinf(back[3])
