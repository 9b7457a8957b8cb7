"""GPU parity of the MXFP4 cache insert (mono_insert_mxfp4) against the oracle.

The bar is bit-exact: every byte of every pool after the insert equals the
oracle's ``insert_rows`` on the same rows, slots and starting pool, written
rows and untouched rows alike.  Slots past the pool must be reported
(DEVERR_SLOT) and not written; negative slots are padding.  The end-to-end
case inserts the decoded tokens' rows and then runs the one-launch step on
the updated pools, checked against the oracle's decode on the oracle's pools.
"""

import numpy as np
import pytest
import torch

from helpers import bf16_bits, bf16_tensor, check_topk_row
from oracle import decode, mxfp4
from workloads import decode_slots, make_workload, new_rows, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_amd as spd

    spd.load_library()
    assert torch.cuda.is_available()
    return spd


def _pools(rng, pages, heads):
    kv = [rng.integers(0, 256, size=(pages, heads, mxfp4.PAGE_BYTES)).astype(np.uint8) for _ in range(2)]
    index = rng.integers(0, 256, size=(pages, mxfp4.PAGE_BYTES)).astype(np.uint8)
    return kv[0], kv[1], index


def _oracle_insert(k_pool, v_pool, index_pool, rows, slots):
    k_new, sk = mxfp4.insert_rows(k_pool, mxfp4.bf16_bits_to_f64(rows["k"]), slots)
    v_new, sv = mxfp4.insert_rows(v_pool, mxfp4.bf16_bits_to_f64(rows["v"]), slots)
    i_new, si = mxfp4.insert_rows(index_pool[:, None, :], mxfp4.bf16_bits_to_f64(rows["index"])[:, None, :], slots)
    assert sk == sv == si
    return k_new, v_new, i_new[:, 0, :], sk


def _gpu_insert(spd, k_pool, v_pool, index_pool, rows, slots, ws, caches=("k", "v", "index")):
    dev = "cuda"
    d = dict(k_pages=torch.from_numpy(k_pool).to(dev), v_pages=torch.from_numpy(v_pool).to(dev),
             index_pages=torch.from_numpy(index_pool).to(dev))
    kw = {}
    for c in caches:
        kw[f"{c}_rows"] = bf16_tensor(rows[c], dev)
        kw[f"{c}_pages"] = d[f"{c}_pages"]
    spd.mono_insert_mxfp4(torch.from_numpy(slots).to(dev), workspace=ws, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in d.items()}


CASES = [
    # name, n, heads, pages, padding fraction, specials
    ("one_row", 1, 1, 1, 0.0, False),
    ("ragged_37", 37, 1, 3, 0.1, False),
    ("two_heads", 300, 2, 5, 0.2, False),
    ("specials", 500, 1, 6, 0.05, True),
    ("all_padding", 20, 1, 2, 1.0, False),
]


@pytest.mark.parametrize("name,n,heads,pages,pad,specials", CASES, ids=[c[0] for c in CASES])
def test_insert_bit_exact(spd, name, n, heads, pages, pad, specials):
    print(f"[insert] {name} n={n} heads={heads} pages={pages}", flush=True)
    rng = np.random.default_rng(sum(map(ord, name)))
    k_pool, v_pool, index_pool = _pools(rng, pages, heads)
    rows = new_rows(7 + n, n, heads, specials=specials)
    slots = rng.permutation(pages * 128)[:n].astype(np.int64)
    slots[rng.random(n) < pad] = -1
    ws = spd.Workspace("cuda")
    got = _gpu_insert(spd, k_pool, v_pool, index_pool, rows, slots, ws)
    assert spd.check_device_errors(ws) == 0
    k_new, v_new, i_new, skipped = _oracle_insert(k_pool, v_pool, index_pool, rows, slots)
    assert skipped == []
    np.testing.assert_array_equal(got["k_pages"], k_new)
    np.testing.assert_array_equal(got["v_pages"], v_new)
    np.testing.assert_array_equal(got["index_pages"], i_new)


def test_slot_past_the_pool_is_reported_and_not_written(spd):
    rng = np.random.default_rng(21)
    k_pool, v_pool, index_pool = _pools(rng, 3, 1)
    rows = new_rows(22, 6, 1)
    slots = np.array([5, 3 * 128, 130, -1, 3 * 128 + 900, 383], dtype=np.int64)
    ws = spd.Workspace("cuda")
    got = _gpu_insert(spd, k_pool, v_pool, index_pool, rows, slots, ws)
    assert spd.check_device_errors(ws) == spd.DEVERR_SLOT
    assert spd.check_device_errors(ws) == 0  # read and cleared
    k_new, v_new, i_new, skipped = _oracle_insert(k_pool, v_pool, index_pool, rows, slots)
    assert skipped == [1, 4]
    np.testing.assert_array_equal(got["k_pages"], k_new)
    np.testing.assert_array_equal(got["v_pages"], v_new)
    np.testing.assert_array_equal(got["index_pages"], i_new)


@pytest.mark.parametrize("caches", [("index",), ("k", "v"), ("v",)], ids=lambda c: "+".join(c))
def test_caches_left_out_are_not_touched(spd, caches):
    rng = np.random.default_rng(23)
    k_pool, v_pool, index_pool = _pools(rng, 4, 2)
    rows = new_rows(24, 50, 2)
    slots = rng.permutation(4 * 128)[:50].astype(np.int64)
    ws = spd.Workspace("cuda")
    got = _gpu_insert(spd, k_pool, v_pool, index_pool, rows, slots, ws, caches=caches)
    assert spd.check_device_errors(ws) == 0
    k_new, v_new, i_new, _ = _oracle_insert(k_pool, v_pool, index_pool, rows, slots)
    np.testing.assert_array_equal(got["k_pages"], k_new if "k" in caches else k_pool)
    np.testing.assert_array_equal(got["v_pages"], v_new if "v" in caches else v_pool)
    np.testing.assert_array_equal(got["index_pages"], i_new if "index" in caches else index_pool)


def test_bad_arguments_are_refused(spd):
    dev = "cuda"
    pages = torch.zeros((2, 1, mxfp4.PAGE_BYTES), dtype=torch.uint8, device=dev)
    rows = torch.zeros((3, 1, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        spd.mono_insert_mxfp4(torch.zeros(3, dtype=torch.int32, device=dev), k_rows=rows, k_pages=pages)
    with pytest.raises(ValueError):
        spd.mono_insert_mxfp4(torch.zeros(3, dtype=torch.int64, device=dev), k_rows=rows)
    with pytest.raises(ValueError):
        spd.mono_insert_mxfp4(torch.zeros(4, dtype=torch.int64, device=dev), k_rows=rows, k_pages=pages)


def _step_matches_oracle(spd, w, d):
    out, sel = spd.mono_sparse_decode_mxfp4(d["index_q"], d["index_pool"], d["q"], d["k_pool"], d["v_pool"],
                                            d["block_table"], d["seq_lens"], w.k, w.scale, T=w.T)
    torch.cuda.synchronize()
    sel, out_bits = sel.cpu().numpy(), bf16_bits(out)
    for i in range(w.N):
        b = i // w.T
        pos = int(w.seq_lens[b]) - w.T + i % w.T
        check_topk_row(sel[i], w, i, w.k)
        ref = decode.decode_one(w.q[i], w.k_pool, w.v_pool, w.block_table[b], pos, w.scale, sel[i])
        vmax = float(np.abs(decode.sequence_rows(w.v_pool, w.block_table[b], pos + 1, 0)).max())
        o = mxfp4.bf16_bits_to_f64(out_bits[i])
        rel = np.linalg.norm(o - ref) / max(np.linalg.norm(ref), 1e-300)
        assert rel <= 5e-3 and np.max(np.abs(o - ref)) <= 1e-2 * vmax, (i, rel)


def test_insert_then_sparse_step(spd):
    # The decoded tokens' K, V and index-key rows go in through the slot
    # mapping, then the step reads them: the step's output must match the
    # oracle's decode over the oracle-inserted pools.
    w = make_workload("insert_step", B=4, T=2, seq_lens=[2, 130, 1000, 3000], bt_width=24, k=300, seed=31)
    rows = new_rows(32, w.N, 1)
    slots = decode_slots(w)
    ws = spd.Workspace("cuda")
    got = _gpu_insert(spd, w.k_pool, w.v_pool, w.index_pool, rows, slots, ws)
    assert spd.check_device_errors(ws) == 0
    w.k_pool, w.v_pool, w.index_pool, skipped = _oracle_insert(w.k_pool, w.v_pool, w.index_pool, rows, slots)
    assert skipped == []
    np.testing.assert_array_equal(got["k_pages"], w.k_pool)
    np.testing.assert_array_equal(got["index_pages"], w.index_pool)
    d = dict(index_q=bf16_tensor(w.index_q, "cuda"), q=bf16_tensor(w.q, "cuda"),
             k_pool=torch.from_numpy(got["k_pages"]).cuda(), v_pool=torch.from_numpy(got["v_pages"]).cuda(),
             index_pool=torch.from_numpy(got["index_pages"]).cuda(),
             block_table=torch.from_numpy(w.block_table).cuda(), seq_lens=torch.from_numpy(w.seq_lens).cuda())
    _step_matches_oracle(spd, w, d)


def test_full_size_decode_insert(spd):
    # One decoded token per request into the pools of the 64-request,
    # 32K-context sparse workload: every pool byte must equal the oracle's.
    w = workload(3)
    print(f"[insert] full size B={w.B} pages={w.num_pages}", flush=True)
    rows = new_rows(33, w.N, 1)
    slots = decode_slots(w)
    ws = spd.Workspace("cuda")
    got = _gpu_insert(spd, w.k_pool, w.v_pool, w.index_pool, rows, slots, ws)
    assert spd.check_device_errors(ws) == 0
    k_new, v_new, i_new, skipped = _oracle_insert(w.k_pool, w.v_pool, w.index_pool, rows, slots)
    assert skipped == []
    np.testing.assert_array_equal(got["k_pages"], k_new)
    np.testing.assert_array_equal(got["v_pages"], v_new)
    np.testing.assert_array_equal(got["index_pages"], i_new)


def test_insert_ties_and_edges_from_golden_blocks(spd):
    """The hand-worked blocks (every e2m1 tie, saturation, signed zeros,
    NaN/inf, subnormals, the largest bf16 exponents), rounded to bf16 and
    shifted by powers of two, so ties occur at many scale bytes."""
    import os

    blocks = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_quantize_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals = [float.fromhex(t) if "p" in t else float(t) for t in line.split()[3:]]
            v = np.zeros(32)
            v[: len(vals)] = vals
            blocks.append(v)
    rows = []
    for v in blocks:
        with np.errstate(over="ignore", invalid="ignore"):
            for j in (-120, -40, -3, 0, 5, 60):
                rows.append(v * 2.0**j)
    rows = np.array(rows)
    n_rows = -(-rows.shape[0] // 4)
    flat = np.zeros((n_rows * 4, 32))
    flat[: rows.shape[0]] = rows
    bits = mxfp4.round_to_bf16_bits(flat.reshape(n_rows, 128))  # out-of-range values become inf blocks
    rng = np.random.default_rng(29)
    pages = -(-n_rows // 128)
    k_pool, v_pool, index_pool = _pools(rng, pages, 1)
    rows_d = {"k": bits[:, None, :], "v": bits[::-1, None, :].copy(), "index": bits}
    slots = rng.permutation(pages * 128)[:n_rows].astype(np.int64)
    ws = spd.Workspace("cuda")
    got = _gpu_insert(spd, k_pool, v_pool, index_pool, rows_d, slots, ws)
    assert spd.check_device_errors(ws) == 0
    k_new, v_new, i_new, _ = _oracle_insert(k_pool, v_pool, index_pool, rows_d, slots)
    np.testing.assert_array_equal(got["k_pages"], k_new)
    np.testing.assert_array_equal(got["v_pages"], v_new)
    np.testing.assert_array_equal(got["index_pages"], i_new)
