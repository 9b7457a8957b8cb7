"""GPU checks of the per-kernel timing hook used by the benchmark."""

import numpy as np
import pytest
import torch

from helpers import to_device
from workloads import make_workload

pytestmark = pytest.mark.gpu


def test_kernel_timer_sees_every_kernel_of_a_step():
    import sparse_paged_decode_amd as spd

    w = make_workload("timer", B=2, T=2, seq_lens=[700, 3000], bt_width=24, k=256, seed=3)
    d = to_device(w)
    with spd.KernelTimer(capacity=64) as kt:
        for _ in range(3):
            sel = spd.mono_index_score_topk(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], w.k, T=w.T)
            spd.mono_pa_decode_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], sel, w.scale,
                                     T=w.T)
        spd.mono_sparse_decode_mxfp4(d["index_q"], d["index_pool"], d["q"], d["k_pool"], d["v_pool"],
                                     d["block_table"], d["seq_lens"], w.k, w.scale, T=w.T)
        torch.cuda.synchronize()
    assert kt.launches == {"index_topk_kernel": 3, "pa_decode_kernel": 3, "sparse_decode_kernel": 1}
    assert all(0 < us < 1e5 for us in kt.mean_us.values())
    # timing off again: launches are not recorded and nothing fails
    sel = spd.mono_index_score_topk(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], w.k, T=w.T)
    torch.cuda.synchronize()
    assert np.all(sel.cpu().numpy()[:, :5] >= 0)
