"""GPU parity at the workloads' full sizes, every query token against the oracle.

Each sparse workload runs in the configuration the benchmark times (one
mono_sparse_decode_mxfp4 launch) and in the two-call form (index call, then
attention call).  For every query token the selection is checked against
the oracle's top-k under the 1e-6 tie band, and the bf16 output against the
oracle's float64 attention over the selection the call returned (relative L2
<= 5e-3, max |err| <= 1e-2 max|V|, per token and over the whole output).
The oracle's dequantised rows of a request are computed once and shared by
its query tokens and by both forms.

Also here: the benchmark's exact sequence (warm-up, then back-to-back steps
over four rotated pool copies with one workspace), each step's output
checked; and "mixing" variants of the dense and sparse workloads at full
shape, with every e8m0 byte fixed at 124 or 127 so that the softmax spreads
over many tokens instead of being one-hot.
"""

import os
import sys

import numpy as np
import pytest
import torch

from helpers import assert_resplit_close, bf16_bits, full_size_check, resplit_bound, to_device
from workloads import workload

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_amd as spd

    spd.load_library()
    assert torch.cuda.is_available()
    return spd


def _both_forms(spd, w):
    d = to_device(w)
    ws = spd.Workspace("cuda")
    out, sel = spd.mono_sparse_decode_mxfp4(d["index_q"], d["index_pool"], d["q"], d["k_pool"], d["v_pool"],
                                            d["block_table"], d["seq_lens"], w.k, w.scale, T=w.T, workspace=ws)
    sel2 = spd.mono_index_score_topk(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], w.k, T=w.T,
                                     workspace=ws)
    out2 = spd.mono_pa_decode_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], sel2,
                                    w.scale, T=w.T, workspace=ws)
    torch.cuda.synchronize()
    assert spd.check_device_errors(ws) == 0
    return (sel.cpu().numpy(), bf16_bits(out)), (sel2.cpu().numpy(), bf16_bits(out2))


@pytest.mark.parametrize("number", [3, 4, 5])
def test_sparse_workload_every_token(spd, number):
    """Workloads 3 (B=64, ctx 32k, top-2048), 4 (B=128, T=4, ctx 16k-64k)
    and 5 (B=8, ctx 256k, top-4096): every query token, both forms."""
    w = workload(number)
    (sel, out), (sel2, out2) = _both_forms(spd, w)
    # the two forms select the same sets
    np.testing.assert_array_equal(np.sort(sel, axis=1), np.sort(sel2, axis=1))
    (rel, frac, n), (rel2, frac2, _) = full_size_check(
        w, [(sel, out, f"{w.name} one launch"), (sel2, out2, f"{w.name} two calls")])
    assert n == w.N
    print(f"{w.name}: {n} query tokens; rel L2 {rel:.2e} / {rel2:.2e}, max err {frac:.2e} / {frac2:.2e} max|V|")


@pytest.mark.parametrize("number,exp", [(2, 124), (2, 127), (3, 124), (3, 127)])
def test_mixing_exponents_full_shape(spd, number, exp):
    """Every e8m0 byte fixed at 124 or 127: logits of standard deviation about
    0.4 or 3, so the softmax mixes many tokens.  Dense workload 2 (every
    token of every request) and sparse workload 3 (one launch)."""
    w = workload(number, exp_range=(exp, exp))
    d = to_device(w)
    ws = spd.Workspace("cuda")
    if w.sparse:
        out, sel = spd.mono_sparse_decode_mxfp4(d["index_q"], d["index_pool"], d["q"], d["k_pool"], d["v_pool"],
                                                d["block_table"], d["seq_lens"], w.k, w.scale, T=w.T, workspace=ws)
        sel_np = sel.cpu().numpy()
    else:
        out = spd.mono_pa_decode_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], None,
                                       w.scale, T=w.T, workspace=ws)
        sel_np = None
    torch.cuda.synchronize()
    assert spd.check_device_errors(ws) == 0
    ((rel, frac, n),) = full_size_check(w, [(sel_np, bf16_bits(out), f"{w.name} e8m0={exp}")])
    assert n == w.N
    print(f"{w.name} e8m0={exp}: rel L2 {rel:.2e}, max err {frac:.2e} max|V|")


@pytest.mark.parametrize("number", [2, 3])
def test_benchmark_sequence(spd, number):
    """The benchmark's own sequence: 5 warm-up and 20 timed steps back to back
    over 4 rotated pool copies with one workspace (bench.py's StepRunner).
    Every step writes its own output buffers; each is checked."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from bench import StepRunner

    w = workload(number)
    run = StepRunner(spd, torch, torch.device("cuda:0"), w, 4)
    n_steps = 25
    outs = [torch.empty_like(run.out) for _ in range(n_steps)]
    sels = [torch.empty_like(run.sel) if w.sparse else None for _ in range(n_steps)]
    for s in range(n_steps):
        run.step(s % run.copies, out=outs[s], sel=sels[s])
    torch.cuda.synchronize()
    for ws in (run.ws, run.ws_pa):
        assert spd.check_device_errors(ws) == 0
    first_sel = sels[0].cpu().numpy() if w.sparse else None
    first_out = bf16_bits(outs[0])
    ((rel, frac, _),) = full_size_check(w, [(first_sel, first_out, f"{w.name} step 0")])
    # Every step reads identical inputs (copies of one pool): the same sets,
    # and outputs that match the checked first step within the bound of a
    # different split of the same candidates (equal, when the splits agree).
    bounds = [resplit_bound(w, i, first_sel[i] if w.sparse else None) for i in range(w.N)]
    same = []
    for s in range(1, n_steps):
        if w.sparse:
            np.testing.assert_array_equal(np.sort(sels[s].cpu().numpy(), axis=1), np.sort(first_sel, axis=1),
                                          err_msg=f"step {s}")
        o = bf16_bits(outs[s])
        same += [assert_resplit_close(o[i], first_out[i], bounds[i], f"step {s} query {i}") for i in range(w.N)]
    print(f"{w.name}: {n_steps} steps; step 0 rel L2 {rel:.2e}, max err {frac:.2e} max|V|; "
          f"{np.mean(same):.4f} of later steps' elements equal to step 0's")
