"""The allocation-free step call (static per-device scratch, no workspace)
against the workspace call, through the C ABI.

Three calls in a row on the same device, each smaller than the one before
(a chunk-local one-token step, a four-token step, a small one-token step):
each must give the selection sets of mono_sparse_decode_mxfp4 on a fresh
workspace, outputs within the bound of a different split of the same
candidates, no device errors, and must match the oracle.  Shapes past the
scratch are refused with MONO_ENOSPC before anything runs.
"""

import numpy as np
import pytest
import torch

from helpers import assert_resplit_close, bf16_bits, check_topk_row, resplit_bound, to_device
from oracle import decode, mxfp4
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_amd as spd

    spd.load_library()
    assert torch.cuda.is_available()
    return spd


def _check_oracle(w, sel_np, out_bits):
    pos = decode.query_positions(w.seq_lens, w.T)
    for i in range(w.N):
        b = i // w.T
        check_topk_row(sel_np[i], w, i, w.k)
        ref = decode.decode_one(w.q[i], w.k_pool, w.v_pool, w.block_table[b], int(pos[i]), w.scale, sel_np[i])
        vmax = float(np.abs(decode.sequence_rows(w.v_pool, w.block_table[b], int(pos[i]) + 1, 0)).max())
        o = mxfp4.bf16_bits_to_f64(out_bits[i])
        rel = np.linalg.norm(o - ref) / np.linalg.norm(ref)
        assert rel <= 5e-3 and np.max(np.abs(o - ref)) <= 1e-2 * vmax, (w.name, i, rel)


def test_noalloc_matches_workspace_call(spd):
    shapes = [
        dict(name="na_big", B=16, T=1, seq_lens=32768, bt_width=256, k=2048, seed=91),
        dict(name="na_t4", B=3, T=4, seq_lens=[700, 5000, 3100], bt_width=40, k=300, seed=92),
        dict(name="na_small", B=2, T=1, seq_lens=[4000, 900], bt_width=40, k=256, seed=93),
    ]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for n, kw in enumerate(shapes):
        name = kw.pop("name")
        w = make_workload(name, exp_range=(124, 127), **kw)
        d = to_device(w)
        out = torch.empty_like(d["q"])
        sel = torch.empty((w.N, w.k), dtype=torch.int32, device="cuda")
        spd.mono_sparse_decode_mxfp4_noalloc(d["index_q"], d["index_pool"], d["q"], d["k_pool"], d["v_pool"],
                                             d["block_table"], d["seq_lens"], w.k, w.scale, out, sel, T=w.T, err=err)
        ws = spd.Workspace("cuda")
        out_ws, sel_ws = spd.mono_sparse_decode_mxfp4(d["index_q"], d["index_pool"], d["q"], d["k_pool"],
                                                      d["v_pool"], d["block_table"], d["seq_lens"], w.k, w.scale,
                                                      T=w.T, workspace=ws)
        torch.cuda.synchronize()
        assert int(err.item()) == 0, (name, int(err.item()))
        assert spd.check_device_errors(ws) == 0
        sel_np, sel_ws_np = sel.cpu().numpy(), sel_ws.cpu().numpy()
        np.testing.assert_array_equal(np.sort(sel_np, axis=1), np.sort(sel_ws_np, axis=1), err_msg=name)
        a, b = bf16_bits(out), bf16_bits(out_ws)
        for i in range(w.N):
            assert_resplit_close(a[i], b[i], resplit_bound(w, i, sel_np[i]), f"{name} query {i}")
        _check_oracle(w, sel_np, a)


def test_noalloc_refuses_shapes_past_the_scratch(spd):
    lib = spd.load_library()
    need = lib.mono_sparse_decode_workspace(128, 4, 1, 512, 2048)
    assert need > spd.NOALLOC_SCRATCH_BYTES
    z = torch.zeros(16, dtype=torch.uint8, device="cuda")
    rc = lib.mono_sparse_decode_mxfp4_noalloc(z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(), 1,
                                              1, z.data_ptr(), 512, z.data_ptr(), 128, 4, 2048, 0.1, z.data_ptr(),
                                              z.data_ptr(), None, None)
    assert rc == spd.MONO_ENOSPC
    assert b"static scratch" in lib.mono_last_error()
