"""The one-launch step under HIP graph capture: captured once, replayed
several times with eager work and synchronisations in between, every
replay checked against the eager result (selection as sets, output to
fp32 summation order).  The call allocates nothing and records no memset,
so it can be captured."""

import numpy as np
import pytest
import torch

from helpers import bf16_bits, to_device
from oracle import mxfp4
from workloads import make_workload

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    import sparse_paged_decode_amd as spd

    w = make_workload("graph", B=3, T=2, seq_lens=[700, 3000, 4100], bt_width=40, k=256, seed=17,
                      exp_range=(124, 127))
    d = to_device(w)
    out = torch.empty_like(d["q"])
    sel = torch.empty((w.N, w.k), dtype=torch.int32, device="cuda")
    ws = spd.Workspace("cuda", spd.sparse_decode_workspace_bytes(w.B, w.T, 1, w.block_table.shape[1], w.k))

    def step():
        spd.mono_sparse_decode_mxfp4(d["index_q"], d["index_pool"], d["q"], d["k_pool"], d["v_pool"],
                                     d["block_table"], d["seq_lens"], w.k, w.scale, T=w.T, out=out,
                                     selected_idx=sel, workspace=ws)

    step()  # eager reference (also sizes the launch before capture)
    torch.cuda.synchronize()
    ref_sel = np.sort(sel.cpu().numpy(), axis=1)
    ref_out = mxfp4.bf16_bits_to_f64(bf16_bits(out))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.zero_()
        sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert spd.check_device_errors(ws) == 0
        np.testing.assert_array_equal(np.sort(sel.cpu().numpy(), axis=1), ref_sel, err_msg=f"replay {rep}")
        o = mxfp4.bf16_bits_to_f64(bf16_bits(out))
        assert np.max(np.abs(o - ref_out)) <= 1e-2 * np.max(np.abs(ref_out)), f"replay {rep}"
        step()  # eager work between replays
        torch.cuda.synchronize()
