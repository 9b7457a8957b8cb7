"""GPU parity of page packing, unpacking and dequantisation (bit-exact)."""

import numpy as np
import pytest
import torch

from oracle import mxfp4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_amd as spd

    spd.load_library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return spd


def _exhaustive_codes_scales(n):
    """Every (even, odd) nibble pair in every byte slot; every scale byte in every slot."""
    pairs = np.array([(a, b) for a in range(16) for b in range(16)], dtype=np.uint8)
    idx = ((np.arange(n * 128 * 64) * 7) % 256).reshape(n, 128, 64)
    codes = np.zeros((n, 128, 128), dtype=np.uint8)
    codes[..., 0::2] = pairs[idx, 0]
    codes[..., 1::2] = pairs[idx, 1]
    scales = ((np.arange(n * 128 * 4) * 11) % 256).astype(np.uint8).reshape(n, 128, 4)
    return codes, scales


def test_pack_unpack_bit_exact(spd):
    codes, scales = _exhaustive_codes_scales(9)
    want = mxfp4.pack(codes, scales)
    dc = torch.from_numpy(codes | (np.arange(codes.size, dtype=np.uint64).reshape(codes.shape) % 16 << 4).astype(np.uint8)).cuda()
    pages = spd.mxfp4_pages_pack(dc, torch.from_numpy(scales).cuda())
    np.testing.assert_array_equal(pages.cpu().numpy(), want)
    c2, s2 = spd.mxfp4_pages_unpack(torch.from_numpy(want).cuda())
    np.testing.assert_array_equal(c2.cpu().numpy(), codes)
    np.testing.assert_array_equal(s2.cpu().numpy(), scales)


def _all_code_exp_pages():
    """Pages in which every (code, e8m0) pair occurs: 16 codes x 256 exponents."""
    codes = np.zeros((8, 128, 128), dtype=np.uint8)
    scales = np.zeros((8, 128, 4), dtype=np.uint8)
    for p in range(8):
        for r in range(128):
            for g in range(4):
                scales[p, r, g] = (p * 512 + r * 4 + g) % 256
    codes[:] = np.arange(128, dtype=np.uint8)[None, None, :] % 16
    # shift the code pattern per row so each code meets each scale in each position
    for r in range(128):
        codes[:, r, :] = (np.arange(128) + r) % 16
    return mxfp4.pack(codes, scales)


def test_dequant_f32_bit_exact_all_codes_and_exponents(spd):
    pages = _all_code_exp_pages()
    want = mxfp4.round_to_f32(mxfp4.dequant(pages))
    got = spd.mxfp4_pages_dequant(torch.from_numpy(pages).cuda()).cpu().numpy()
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok].view(np.uint32), want[ok].view(np.uint32))  # keeps -0.0


def test_dequant_bf16_conversion_bit_exact(spd):
    """The conversion the scoring and attention kernels use, on all 16 x 256 pairs."""
    pages = _all_code_exp_pages()
    want = mxfp4.round_to_bf16_bits(mxfp4.dequant(pages))
    got = spd.mxfp4_pages_dequant_bf16(torch.from_numpy(pages).cuda()).cpu().view(torch.int16).numpy().view(np.uint16)
    nan_w = (want & 0x7F80) == 0x7F80
    nan_w &= (want & 0x7F) != 0
    nan_g = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    e = mxfp4.unpack(pages)[1]
    exps = np.repeat(e, 32, axis=-1)
    # report the exponent range where the conversion is exact
    mismatch = (got != want) & ~(nan_w & nan_g)
    bad_exps = np.unique(exps[mismatch])
    assert mismatch.sum() == 0, f"bf16 conversion differs at e8m0 bytes {bad_exps.tolist()[:20]}"


def test_zero_pages_is_noop(spd):
    lib = spd.load_library()
    assert lib.mxfp4_pages_pack(None, None, None, 0, None) == 0
    assert lib.mxfp4_pages_dequant(None, None, 0, None) == 0
