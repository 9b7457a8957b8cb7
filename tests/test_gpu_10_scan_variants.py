"""The index scan on the matrix cores and on the VALU (benchmark kernels).

Both variants score every token a request's query sees and count the
scores in 2048 histogram bins of the top score-key bits.  Pinned against
the oracle's exact scores: every request's counts sum to its length, and
the per-bin counts match the oracle's fp32 scores' bins except for tokens
whose exact score lies within a few fp32 units of a bin edge (the two
variants and the oracle sum the 128 products in different orders).
"""

import numpy as np
import pytest
import torch

from helpers import to_device
from oracle import decode
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_amd as spd

    spd.load_library()
    assert torch.cuda.is_available()
    return spd


def _key_bins(scores):
    """Top 11 bits of the order-preserving key of fp32 scores (NaN sorts lowest)."""
    b = np.asarray(scores, dtype=np.float32).view(np.uint32).astype(np.uint64)
    key = np.where(b & 0x80000000, ~b & 0xFFFFFFFF, b | 0x80000000)
    key = np.where(np.isnan(np.asarray(scores, dtype=np.float32)), 0, key)
    return (key >> 21).astype(np.int64)


@pytest.mark.parametrize("variant", [0, 1], ids=["mfma", "valu"])
def test_scan_variant_histograms(spd, variant):
    lens = [1, 127, 128, 129, 3000, 4096]
    w = make_workload("scanvar", B=len(lens), T=1, seq_lens=lens, bt_width=32, k=16, seed=91, exp_range=(124, 127))
    d = to_device(w)
    print(f"[scan] variant {variant}", flush=True)
    hist, err = spd.bench_scan(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], 8, variant)
    torch.cuda.synchronize()
    assert int(err.cpu()[0]) == 0
    hist = hist.cpu().numpy().astype(np.int64)
    for b, L in enumerate(lens):
        assert hist[b].sum() == L, f"request {b}: counts"
        exact = decode.index_scores(w.index_q[b], w.index_pool, w.block_table[b], L - 1)
        want = np.bincount(_key_bins(exact.astype(np.float32)), minlength=2048)
        # a token can change bins only if its score sits next to a bin edge
        lo = _key_bins((exact * (1 - 1e-6)).astype(np.float32))
        hi = _key_bins((exact * (1 + 1e-6)).astype(np.float32))
        loose = int(np.sum(lo != hi))
        assert np.abs(hist[b] - want).sum() <= 2 * loose, f"request {b}: bins"
