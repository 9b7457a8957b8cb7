"""Pins of the oracle's fp8 (e4m3) cache pages and of the decode math on them.

Checked against: hand-worked e4m3 values (``golden/e4m3_values.txt``),
torch's ``float8_e4m3fn`` conversion of all 256 codes, single-byte pages
for the row geometry, one-hot index pages for the scores, closed forms of
the per-tensor K / V scales, and torch float64 attention over rows gathered
independently through torch's fp8 conversion.
"""

import os

import numpy as np
import pytest
import torch

from oracle import decode, fp8, mxfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    out = []
    with open(os.path.join(GOLDEN, "e4m3_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()
                out.append((int(code, 16), float(val)))
    return out


@pytest.mark.parametrize("code,val", _golden(), ids=lambda x: f"{x:02X}" if isinstance(x, int) else "")
def test_e4m3_golden(code, val):
    got = float(fp8.e4m3_value(code))
    if np.isnan(val):
        assert np.isnan(got)
    else:
        assert got == val and np.signbit(got) == np.signbit(val)


def test_e4m3_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.e4m3_value(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_positive_codes_increase_and_negatives_mirror():
    pos = fp8.e4m3_value(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0
    neg = fp8.e4m3_value(np.arange(0x80, 0xFF))
    np.testing.assert_array_equal(neg, -pos)


def test_row_geometry_single_bytes():
    rng = np.random.default_rng(3)
    for _ in range(20):
        r, i = rng.integers(0, 128, size=2)
        page = np.zeros(fp8.PAGE_BYTES, dtype=np.uint8)
        page[128 * r + i] = 0x38  # 1.0
        v = fp8.dequant(page)
        assert v.shape == (128, 128) and v[r, i] == 1.0 and np.count_nonzero(v) == 1
    with pytest.raises(ValueError):
        fp8.dequant(np.zeros(8704, dtype=np.uint8))


def test_sequence_rows_dispatches_on_page_size():
    with pytest.raises(ValueError):
        decode.sequence_rows(np.zeros((2, 1000), dtype=np.uint8), np.array([0, 1]), 10)
    # an fp8 pool reads as fp8, an MXFP4 pool as MXFP4
    z8 = np.zeros((1, fp8.PAGE_BYTES), dtype=np.uint8)
    z8[0, 0] = 0x40  # 2.0 at token 0, element 0
    assert decode.sequence_rows(z8, np.array([0]), 1)[0, 0] == 2.0
    z4 = np.zeros((1, mxfp4.PAGE_BYTES), dtype=np.uint8)
    z4[0, 0] = 0x07  # e2m1 code 7 = 6.0 in element 0
    z4[0, mxfp4.DATA_REGION] = 127
    assert decode.sequence_rows(z4, np.array([0]), 1)[0, 0] == 6.0


def test_index_scores_one_hot_fp8_pages():
    # Token j's index row holds a single 1.0 at element d_j: its score is
    # index_q[d_j] exactly, through a permuted block table.
    rng = np.random.default_rng(4)
    P, n = 4, 400
    pool = np.zeros((P, fp8.PAGE_BYTES), dtype=np.uint8)
    bt = rng.permutation(P).astype(np.int64)
    d = rng.integers(0, 128, size=n)
    for j in range(n):
        pool[bt[j // 128], 128 * (j % 128) + d[j]] = 0x38
    iq = mxfp4.round_to_bf16_bits(rng.standard_normal(128))
    s = decode.index_scores(iq, pool, bt, n - 1)
    np.testing.assert_array_equal(s, mxfp4.bf16_bits_to_f64(iq)[d])


def _fp8_pools(rng, P):
    codes = rng.integers(0, 0x7F, size=(2, P, 1, fp8.PAGE_BYTES)) | (rng.integers(0, 2, size=(2, P, 1, fp8.PAGE_BYTES)) << 7)
    exp_cap = (codes & 0x78) > 0x50  # keep magnitudes small: exponent field <= 10
    codes = np.where(exp_cap, codes & 0x87 | 0x40, codes)
    return codes[0].astype(np.uint8), codes[1].astype(np.uint8)


def test_tensor_scales_closed_forms():
    rng = np.random.default_rng(5)
    kp, vp = _fp8_pools(rng, 3)
    bt = np.array([2, 0, 1])
    q = mxfp4.round_to_bf16_bits(rng.standard_normal((16, 128)))
    base = decode.decode_one(q, kp, vp, bt, 300, 0.05)
    # k_scale multiplies every logit like the softmax scale does
    np.testing.assert_allclose(decode.decode_one(q, kp, vp, bt, 300, 0.05, k_scale=2.0),
                               decode.decode_one(q, kp, vp, bt, 300, 0.1), rtol=1e-12, atol=1e-12)
    # v_scale multiplies the output
    np.testing.assert_allclose(decode.decode_one(q, kp, vp, bt, 300, 0.05, v_scale=0.375), 0.375 * base,
                               rtol=1e-12, atol=1e-12)


def test_attention_matches_torch_on_fp8_rows():
    rng = np.random.default_rng(6)
    kp, vp = _fp8_pools(rng, 4)
    bt = np.array([3, 1, 0, 2])
    q = mxfp4.round_to_bf16_bits(rng.standard_normal((16, 128)))
    pos, ks, vs, scale = 450, 0.25, 0.5, 1 / np.sqrt(128)
    sel = rng.permutation(pos + 1)[:100]
    got = decode.decode_one(q, kp, vp, bt, pos, scale, sel, k_scale=ks, v_scale=vs)

    def rows(pool):  # independent gather: torch fp8 view of [page, 128, 128]
        t = torch.from_numpy(pool[:, 0]).view(torch.float8_e4m3fn).to(torch.float64).reshape(-1, 128, 128)
        return torch.stack([t[bt[j // 128], j % 128] for j in sel])

    qt = torch.from_numpy(mxfp4.bf16_bits_to_f64(q))
    z = scale * (qt @ (ks * rows(kp)).T)
    ref = torch.softmax(z, dim=-1) @ (vs * rows(vp))
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)
