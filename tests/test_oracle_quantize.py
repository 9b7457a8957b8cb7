"""Pins of the oracle's MXFP4 quantisation and cache insert.

The pages name the MXFP4 cache writer and its int64 page-128 slot mapping
but print no rounding rule; the oracle takes the OCP Microscaling v1.0
conversion.  Its pins: hand-worked blocks (``golden/mxfp4_quantize_blocks.txt``,
ties, saturation, zero, NaN/inf, both clamps), exact round trips of values
already on the MXFP4 grid through the pinned ``dequant``, the power-of-two
scaling and sign symmetries, the rounding-error bound of e2m1, monotonicity,
and the slot geometry of the insert checked through the pinned ``unpack``.
"""

import os

import numpy as np
import pytest

from oracle import mxfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MAGS = np.array(mxfp4.E2M1_MAGNITUDES)


def _golden_blocks():
    out = []
    with open(os.path.join(GOLDEN, "mxfp4_quantize_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, byte, codes, *vals = line.split()
            v = np.zeros(32)
            v[: len(vals)] = [float.fromhex(t) if "p" in t else float(t) for t in vals]
            out.append((name, int(byte), [int(c, 16) for c in codes], v))
    return out


@pytest.mark.parametrize("name,byte,codes,v", _golden_blocks(), ids=lambda x: x if isinstance(x, str) else "")
def test_golden_blocks(name, byte, codes, v):
    got_codes, got_byte = mxfp4.quantize_block(v)
    assert got_byte == byte
    assert list(got_codes) == codes


def _grid_codes(rng, n_blocks):
    """Random e2m1 codes whose blocks each hold a code of magnitude 4 or 6."""
    codes = rng.integers(0, 16, size=(n_blocks, 32)).astype(np.uint8)
    pos = rng.integers(0, 32, size=n_blocks)
    top = rng.choice(np.array([6, 7, 14, 15], dtype=np.uint8), size=n_blocks)
    codes[np.arange(n_blocks), pos] = top
    return codes


def test_grid_values_round_trip_exactly():
    # A block already on the MXFP4 grid with magnitude 4 or 6 present has
    # floor(log2 max) = byte - 127 + 2, so the conversion must give back its
    # own codes and scale byte (including -0.0 as code 8).
    rng = np.random.default_rng(11)
    codes = _grid_codes(rng, 400)
    bytes_ = rng.integers(1, 251, size=400)
    for c, b in zip(codes, bytes_):
        v = mxfp4.e2m1_value(c) * mxfp4.e8m0_value(b)
        got_c, got_b = mxfp4.quantize_block(v)
        assert got_b == b
        np.testing.assert_array_equal(got_c, c)


def test_rows_round_trip_through_pinned_dequant():
    # Pages built from grid codes, dequantised by the pinned dequant, then
    # quantised row by row: element i of a row must use scale byte i // 32.
    rng = np.random.default_rng(12)
    codes = _grid_codes(rng, 2 * 128 * 4).reshape(2, 128, 128)
    scales = rng.integers(100, 150, size=(2, 128, 4)).astype(np.uint8)
    rows = mxfp4.dequant(mxfp4.pack(codes, scales))
    got_c, got_s = mxfp4.quantize_rows(rows)
    np.testing.assert_array_equal(got_c, codes)
    np.testing.assert_array_equal(got_s, scales)


def _random_blocks(rng, n):
    scale = 2.0 ** rng.integers(-20, 20, size=(n, 1))
    v = rng.standard_normal((n, 32)) * scale
    v[rng.random((n, 32)) < 0.05] = 0.0
    return v


def test_power_of_two_scaling_shifts_only_the_byte():
    rng = np.random.default_rng(13)
    for v in _random_blocks(rng, 200):
        c, b = mxfp4.quantize_block(v)
        for j in (-7, -1, 1, 5):
            c2, b2 = mxfp4.quantize_block(v * 2.0**j)
            assert b2 == b + j
            np.testing.assert_array_equal(c2, c)


def test_negation_flips_only_the_sign_bits():
    rng = np.random.default_rng(14)
    for v in _random_blocks(rng, 200):
        c, b = mxfp4.quantize_block(v)
        c2, b2 = mxfp4.quantize_block(-v)
        assert b2 == b
        np.testing.assert_array_equal(c2, c ^ 8)


def test_rounding_error_bound_and_monotonicity():
    # With s = byte - 127 and q = |v| / 2^s: the largest q lies in [4, 8);
    # q <= 6 is off its e2m1 value by at most half the local spacing (0.25
    # below 2, 0.5 in [2, 4), 1 in [4, 6]); q > 6 gives 6; and larger |v|
    # never gets a smaller magnitude.
    rng = np.random.default_rng(15)
    for v in _random_blocks(rng, 300):
        c, b = mxfp4.quantize_block(v)
        q = np.abs(v) / 2.0 ** (int(b) - 127)
        d = MAGS[c & 7]
        assert 4.0 <= q.max() < 8.0
        half = np.where(q < 2, 0.25, np.where(q < 4, 0.5, 1.0))
        inside = q <= 6
        assert np.all(np.abs(q - d)[inside] <= half[inside])
        assert np.all(d[~inside] == 6.0)
        order = np.argsort(q, kind="stable")
        assert np.all(np.diff(d[order]) >= 0)
        np.testing.assert_array_equal(c >> 3, np.signbit(v).astype(np.uint8))


def _pool(rng, pages, heads):
    return rng.integers(0, 256, size=(pages, heads, mxfp4.PAGE_BYTES)).astype(np.uint8)


def test_insert_writes_row_slot_mod_128_of_page_slot_div_128():
    rng = np.random.default_rng(16)
    pages, heads, n = 5, 2, 40
    pool = _pool(rng, pages, heads)
    rows = rng.standard_normal((n, heads, 128)) * 3
    slots = rng.permutation(pages * 128)[:n].astype(np.int64)
    slots[3] = -1  # padding: skipped
    slots[7] = pages * 128 + 5  # past the pool: skipped and reported
    new, skipped = mxfp4.insert_rows(pool, rows, slots)
    assert skipped == [7]
    want_c, want_s = mxfp4.quantize_rows(rows)
    new_c, new_s = mxfp4.unpack(new)
    old_c, old_s = mxfp4.unpack(pool)
    written = np.zeros((pages, heads, 128), dtype=bool)
    for t, s in enumerate(slots):
        if s < 0 or s >= pages * 128:
            continue
        p, r = divmod(int(s), 128)
        written[p, :, r] = True
        for h in range(heads):
            np.testing.assert_array_equal(new_c[p, h, r], want_c[t, h])
            np.testing.assert_array_equal(new_s[p, h, r], want_s[t, h])
    np.testing.assert_array_equal(new_c[~written], old_c[~written])
    np.testing.assert_array_equal(new_s[~written], old_s[~written])
    # the input pool is not modified
    np.testing.assert_array_equal(mxfp4.unpack(pool)[0], old_c)


def test_insert_then_dequant_gives_grid_values_back():
    rng = np.random.default_rng(17)
    codes = _grid_codes(rng, 6 * 4).reshape(6, 1, 128)
    scales = rng.integers(110, 140, size=(6, 1, 4)).astype(np.uint8)
    want = mxfp4.e2m1_value(codes) * np.repeat(mxfp4.e8m0_value(scales), 32, axis=-1)
    pool = np.zeros((2, 1, mxfp4.PAGE_BYTES), dtype=np.uint8)
    slots = np.array([0, 127, 128, 200, 255, 1], dtype=np.int64)
    new, skipped = mxfp4.insert_rows(pool, want, slots)
    assert skipped == []
    got = mxfp4.dequant(new)
    for t, s in enumerate(slots):
        np.testing.assert_array_equal(got[s // 128, 0, s % 128], want[t, 0])


def test_insert_of_nothing_changes_nothing():
    rng = np.random.default_rng(18)
    pool = _pool(rng, 2, 1)
    new, skipped = mxfp4.insert_rows(pool, np.zeros((3, 1, 128)), np.array([-1, -1, -5]))
    assert skipped == []
    np.testing.assert_array_equal(new, pool)
