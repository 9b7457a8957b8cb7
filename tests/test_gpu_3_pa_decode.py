"""GPU parity of paged MXFP4 decode attention against the oracle.

Tolerance: relative L2 <= 5e-3 over the output and max |err| <= 1e-2 max|V|.
Besides the seeded workloads, "mixing" variants with small fixed exponents
(logit std ~0.4 and ~3) make the softmax spread over many tokens, so a wrong
P.V mix cannot hide behind a one-hot softmax.
"""

import numpy as np
import pytest
import torch

from helpers import assert_attention_close, assert_resplit_close, bf16_bits, max_abs_v, resplit_bound, to_device
from oracle import decode, mxfp4
from workloads import make_workload, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_amd as spd

    spd.load_library()
    assert torch.cuda.is_available()
    return spd


def _run(spd, w, sel=None, d=None, kv_heads=1):
    d = d or to_device(w)
    ws = spd.Workspace("cuda")
    sel_t = None if sel is None else torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
    out = spd.mono_pa_decode_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], sel_t,
                                   w.scale, T=w.T, workspace=ws)
    torch.cuda.synchronize()
    assert spd.check_device_errors(ws) == 0
    # the same workspace serves the next call: split counters were reset
    again = spd.mono_pa_decode_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], sel_t,
                                     w.scale, T=w.T, workspace=ws)
    assert torch.equal(again, out)
    return out


def _check(spd, w, sel=None, what=""):
    out = _run(spd, w, sel)
    ref = decode.pa_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, w.T, w.scale, sel)
    vmax = max_abs_v(w, w.seq_lens)
    return assert_attention_close(out, ref, vmax, what)


DENSE = [
    # name, B, T, seq_lens, bt_width, exps
    ("one_token", 1, 1, [1], 1, (122, 132)),
    ("tiny_dense", 1, 1, [256], 2, (122, 132)),
    ("ragged", 3, 1, [5, 129, 1000], 8, (122, 132)),
    ("mix124", 2, 1, [700, 1500], 12, (124, 124)),
    ("mix127", 2, 1, [700, 1500], 12, (127, 127)),
    ("multi_token", 3, 4, [4, 260, 1111], 9, (124, 126)),
    ("long_splits", 2, 1, [9000, 6001], 71, (123, 127)),
]


@pytest.mark.parametrize("name,B,T,lens,W,exps", DENSE, ids=[c[0] for c in DENSE])
def test_dense_small(spd, name, B, T, lens, W, exps):
    w = make_workload(name, B=B, T=T, seq_lens=lens, bt_width=W, k=0, seed=sum(map(ord, name)), exp_range=exps)
    _check(spd, w, None, name)


@pytest.mark.parametrize("exps", [(122, 132), (124, 124), (127, 127)])
def test_sparse_small_with_oracle_selection(spd, exps):
    w = make_workload("sp", B=3, T=2, seq_lens=[300, 2000, 4100], bt_width=33, k=200, seed=31, exp_range=exps)
    sel = decode.index_topk(w.index_q, w.index_pool, w.block_table, w.seq_lens, w.T, w.k)
    _check(spd, w, sel, f"sparse {exps}")


def test_sparse_list_with_invalid_entries(spd):
    """Entries < 0 or past the position are skipped; order does not matter."""
    w = make_workload("inv", B=2, T=1, seq_lens=[500, 900], bt_width=8, k=0, seed=4, exp_range=(124, 126))
    rng = np.random.default_rng(1)
    sel = np.full((2, 96), -1, dtype=np.int64)
    sel[0, :40] = rng.permutation(500)[:40]
    sel[0, 50:60] = 500 + np.arange(10)  # past the position
    sel[1, 10:90] = rng.permutation(900)[:80]
    sel[1, 5] = -7
    _check(spd, w, sel, "invalid entries")


def test_sparse_all_invalid_gives_zero(spd):
    w = make_workload("zero", B=1, T=1, seq_lens=[100], bt_width=1, k=0, seed=2)
    sel = np.full((1, 64), -1)
    sel[0, 3] = 150
    out = _run(spd, w, sel)
    assert torch.count_nonzero(out.float()) == 0


def test_sparse_all_valid_equals_dense(spd):
    w = make_workload("eqd", B=2, T=2, seq_lens=[333, 600], bt_width=5, k=0, seed=12, exp_range=(124, 127))
    pos = decode.query_positions(w.seq_lens, w.T)
    sel = np.full((4, 640), -1)
    for i, p in enumerate(pos):
        sel[i, : p + 1] = np.random.default_rng(i).permutation(p + 1)
    dense = bf16_bits(_run(spd, w, None)).astype(np.int64)
    sparse = bf16_bits(_run(spd, w, sel)).astype(np.int64)
    # same math, different token order and split: equal up to fp32 rounding order
    a = mxfp4.bf16_bits_to_f64(dense.astype(np.uint16))
    b = mxfp4.bf16_bits_to_f64(sparse.astype(np.uint16))
    assert np.max(np.abs(a - b)) <= 1e-2 * np.max(np.abs(a))


def test_nan_poison_in_masked_rows(spd):
    """NaN scales (e8m0 0xFF) in rows past the sequence end must not reach the output."""
    w = make_workload("poison", B=2, T=2, seq_lens=[200, 333], bt_width=3, k=0, seed=14, exp_range=(124, 127))
    clean = _run(spd, w, None)
    for b, L in enumerate(w.seq_lens):
        last = w.block_table[b, (L - 1) // 128]
        r0 = L % 128
        if r0:
            w.k_pool[last, 0, 8192 + 4 * r0 :] = 0xFF
            w.v_pool[last, 0, 8192 + 4 * r0 :] = 0xFF
    poisoned = _run(spd, w, None)
    assert torch.isfinite(poisoned.float()).all()
    assert torch.equal(poisoned, clean)


def test_kv_heads_two(spd):
    w = make_workload("h2", B=2, T=1, seq_lens=[260, 700], bt_width=6, k=0, seed=3, exp_range=(124, 127))
    rng = np.random.default_rng(5)
    k2 = rng.integers(0, 256, size=(w.num_pages, 2, 8704), dtype=np.uint8)
    v2 = rng.integers(0, 256, size=(w.num_pages, 2, 8704), dtype=np.uint8)
    k2[..., 8192:] = rng.integers(124, 128, size=(w.num_pages, 2, 512))
    v2[..., 8192:] = rng.integers(124, 128, size=(w.num_pages, 2, 512))
    q2 = mxfp4.round_to_bf16_bits(rng.standard_normal((2, 32, 128)))
    w.k_pool, w.v_pool, w.q = k2, v2, q2
    out = _run(spd, w)
    for h in range(2):
        ref = decode.pa_decode(q2[:, 16 * h : 16 * h + 16], k2, v2, w.block_table, w.seq_lens, 1, w.scale, None, head=h)
        vmax = max(float(np.abs(decode.sequence_rows(v2, w.block_table[b], int(w.seq_lens[b]), h)).max()) for b in range(2))
        assert_attention_close(out[:, 16 * h : 16 * h + 16], ref, vmax, f"head {h}")


def test_page_permutation_invariance(spd):
    w = make_workload("perm", B=2, T=1, seq_lens=[1000, 777], bt_width=8, k=0, seed=21, exp_range=(124, 127))
    a = _run(spd, w)
    perm = np.random.default_rng(0).permutation(w.num_pages)
    inv = np.argsort(perm)
    w.block_table = np.where(w.block_table >= 0, inv[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    w.k_pool, w.v_pool = w.k_pool[perm], w.v_pool[perm]
    b = _run(spd, w)
    assert torch.equal(a, b)


def test_bad_page_id_is_flagged(spd):
    w = make_workload("badp", B=2, T=1, seq_lens=[300, 300], bt_width=3, k=0, seed=9)
    d = to_device(w)
    d["block_table"][0, 2] = -5
    ws = spd.Workspace("cuda")
    spd.mono_pa_decode_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], None, w.scale,
                             workspace=ws)
    assert spd.check_device_errors(ws) & spd.DEVERR_PAGE_ID


def test_workload_1_tiny_dense_full(spd):
    w = workload(1)
    _check(spd, w, None, "tiny dense")


def test_workload_2_dense_full(spd):
    w = workload(2)
    _check(spd, w, None, "dense b32 ctx8k")




def test_split_count_invariance(spd):
    """The same 256 candidates of one query token as a list of 256 entries
    (one split: no merge), and spread with -1 padding over lists of 4096 and
    8192 entries (16 and 32 splits of 256 entries, merged).  The merge is
    exact up to fp32 rounding; what changes with the split count is the bf16
    rounding of each probability, taken relative to its split's running
    maximum.  So the three outputs must agree within the bound that rounding
    implies (helpers.resplit_bound), and each must match the oracle."""
    w = make_workload("splits", B=1, T=1, seq_lens=[8192], bt_width=64, k=0, seed=71, exp_range=(124, 127))
    d = to_device(w)
    rng = np.random.default_rng(72)
    cand = np.sort(rng.choice(8192, size=256, replace=False)).astype(np.int32)
    outs = []
    for k in (256, 4096, 8192):
        row = np.full((1, k), -1, dtype=np.int32)
        row[0, :: k // 256] = cand
        sel = torch.from_numpy(row).cuda()
        out = spd.mono_pa_decode_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], sel,
                                       w.scale, workspace=spd.Workspace("cuda"))
        torch.cuda.synchronize()
        bits = bf16_bits(out)
        o = mxfp4.bf16_bits_to_f64(bits)
        ref = decode.pa_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, 1, w.scale, row)
        assert np.linalg.norm(o - ref) <= 5e-3 * np.linalg.norm(ref), k
        outs.append(bits)
    bound = resplit_bound(w, 0, cand)
    for n, o in enumerate(outs[1:]):
        same = assert_resplit_close(o[0], outs[0][0], bound, f"{(4096, 8192)[n]} entries vs 256")
        print(f"split-count invariance: {same:.3f} of the elements identical")
