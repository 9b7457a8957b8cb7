"""GPU parity of index scoring + top-k against the oracle.

Small cases compare every query token; the full-size workloads (the ones the
benchmark times, in the same launch configuration) compare sampled query
tokens one by one.
"""

import numpy as np
import pytest
import torch

from helpers import check_topk_row, to_device
from oracle import decode, mxfp4
from workloads import make_workload, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_amd as spd

    spd.load_library()
    assert torch.cuda.is_available()
    return spd


def _run(spd, w, k, **kw):
    d = to_device(w)
    ws = spd.Workspace("cuda")
    sel, scores = spd.mono_index_score_topk(
        d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], k, T=w.T, return_scores=True,
        workspace=ws, **kw)
    torch.cuda.synchronize()
    assert spd.check_device_errors(ws) == 0
    # the same workspace serves the next call: counters and histograms were reset
    again = spd.mono_index_score_topk(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], k, T=w.T,
                                      workspace=ws, **kw)
    np.testing.assert_array_equal(np.sort(again.cpu().numpy(), axis=1), np.sort(sel.cpu().numpy(), axis=1))
    return sel.cpu().numpy(), scores.cpu().numpy()


SMALL = [
    # name, B, T, seq_lens, bt_width, k
    ("one_page_k_lt_n", 1, 1, [100], 1, 10),
    ("k_ge_valid", 2, 1, [50, 129], 2, 200),
    ("k_one", 3, 1, [1, 128, 700], 6, 1),
    ("ragged_multi_token", 4, 4, [4, 300, 1000, 2049], 17, 37),
    ("several_chunks", 2, 1, [5000, 4097], 40, 700),
    ("t3_group", 2, 3, [640, 3001], 24, 250),
    ("t6_two_groups", 2, 6, [900, 2300], 18, 128),
    # score rows longer than 64K: the slice-and-resolve selection
    ("wide_table_slices", 2, 1, [3000, 9000], 520, 700),
    ("wide_table_slices_t2", 2, 2, [5000, 9100], 520, 300),
]


@pytest.mark.parametrize("name,B,T,lens,W,k", SMALL, ids=[c[0] for c in SMALL])
def test_topk_small(spd, name, B, T, lens, W, k):
    w = make_workload(name, B=B, T=T, seq_lens=lens, bt_width=W, k=k, seed=sum(map(ord, name)))
    sel, scores = _run(spd, w, k)
    for i in range(w.N):
        check_topk_row(sel[i], w, i, k)
        # the reported scores are the fp32 scores of the reported tokens
        b = i // T
        pos = int(w.seq_lens[b]) - T + i % T
        n = min(k, pos + 1)
        s = decode.index_scores(w.index_q[i], w.index_pool, w.block_table[b], pos)
        # fp32 accumulation of 128 exact products: |err| <= 128 * 2^-24 * sum |products|
        rows = decode.sequence_rows(w.index_pool, w.block_table[b], pos + 1)
        mag = np.abs(rows) @ np.abs(mxfp4.bf16_bits_to_f64(w.index_q[i]))
        j = sel[i, :n]
        assert np.all(np.abs(scores[i, :n] - s[j]) <= 128 * 2.0**-24 * mag[j])
        assert np.all(np.isnan(scores[i, n:]))


def test_topk_scale_stress(spd):
    """Wide e8m0 range (as the long-context workload uses)."""
    w = make_workload("wide", B=2, T=1, seq_lens=[3000, 2222], bt_width=24, k=300, seed=77, exp_range=(110, 140))
    sel, _ = _run(spd, w, 300)
    for i in range(w.N):
        check_topk_row(sel[i], w, i, 300)


def test_topk_all_equal_scores_overflow_path(spd):
    """Every score equal: the candidate list overflows and ties go to the lowest indices."""
    w = make_workload("eq", B=1, T=1, seq_lens=[9000], bt_width=71, k=1000, seed=5)
    codes = np.full((w.num_pages, 128, 128), 2, dtype=np.uint8)
    w.index_pool = mxfp4.pack(codes, np.full((w.num_pages, 128, 4), 127, dtype=np.uint8))
    sel, _ = _run(spd, w, 1000)
    assert sorted(sel[0].tolist()) == list(range(1000))


def test_topk_many_ties_in_candidate_list(spd):
    """A few distinct score values: exact ties at the threshold, candidates fit the list."""
    w = make_workload("ties", B=1, T=1, seq_lens=[3000], bt_width=24, k=777, seed=6)
    rng = np.random.default_rng(0)
    codes = np.zeros((w.num_pages, 128, 128), dtype=np.uint8)
    codes[:, :, 0] = rng.integers(0, 8, size=(w.num_pages, 128))  # score = iq[0] * value
    w.index_pool = mxfp4.pack(codes, np.full((w.num_pages, 128, 4), 127, dtype=np.uint8))
    w.index_q[:, 0] = mxfp4.round_to_bf16_bits(np.array([1.0]))[0]
    sel, _ = _run(spd, w, 777)
    check_topk_row(sel[0], w, 0, 777)
    ref = decode.topk(decode.index_scores(w.index_q[0], w.index_pool, w.block_table[0], 2999), 777)
    assert sorted(sel[0].tolist()) == sorted(ref.tolist())  # lowest-index tie-break, exactly


@pytest.mark.parametrize("L,W,k", [(3000, 24, 776), (60000, 470, 2048)], ids=["select_row", "slice_rows"])
def test_topk_exact_ties_few_per_value(spd, L, W, k):
    """512 distinct score values (v0 + v1/16 + v2/256 over e2m1 magnitudes),
    each held by a few to a hundred tokens: the last radix level ends in a
    small bin of exact ties, which goes to the lowest indices."""
    w = make_workload("ties512", B=1, T=1, seq_lens=[L], bt_width=W, k=k, seed=7)
    rng = np.random.default_rng(1)
    codes = np.zeros((w.num_pages, 128, 128), dtype=np.uint8)
    codes[:, :, 0:3] = rng.integers(0, 8, size=(w.num_pages, 128, 3))
    w.index_pool = mxfp4.pack(codes, np.full((w.num_pages, 128, 4), 127, dtype=np.uint8))
    w.index_q[:, :] = 0
    w.index_q[:, 0:3] = mxfp4.round_to_bf16_bits(np.array([1.0, 1.0 / 16, 1.0 / 256]))
    sel, scores = _run(spd, w, k)
    s = decode.index_scores(w.index_q[0], w.index_pool, w.block_table[0], L - 1)
    ref = decode.topk(s, k)
    assert sorted(sel[0].tolist()) == sorted(ref.tolist())  # lowest-index tie-break, exactly
    assert np.array_equal(scores[0], s[sel[0]])  # every sum is exact in fp32


def test_topk_repeat_calls_deterministic(spd):
    w = make_workload("rep", B=3, T=2, seq_lens=[3000, 5000, 4100], bt_width=40, k=512, seed=8)
    a, _ = _run(spd, w, 512)
    b, _ = _run(spd, w, 512)
    np.testing.assert_array_equal(np.sort(a, axis=1), np.sort(b, axis=1))


def test_topk_bad_page_id_is_flagged_not_dereferenced(spd):
    w = make_workload("bad", B=2, T=1, seq_lens=[300, 300], bt_width=3, k=16, seed=9)
    d = to_device(w)
    d["block_table"][1, 1] = 10**6
    ws = spd.Workspace("cuda")
    spd.mono_index_score_topk(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], 16, workspace=ws)
    assert spd.check_device_errors(ws) & spd.DEVERR_PAGE_ID


# Many query tokens: more filter slices than two rounds of the resident
# workgroups, so each token's top k is taken by one workgroup.
MANY = [
    ("many_queries_t1", 300, 1, (100, 3000), 100, 300),
    ("many_queries_t2", 150, 2, (100, 5000), 100, 500),
    # more tokens above the threshold bin than the LDS staging holds (2048):
    # each lane writes its own
    ("many_queries_k_over_2048", 300, 1, (2000, 6000), 100, 2500),
]


@pytest.mark.parametrize("name,B,T,lens,W,k", MANY, ids=[c[0] for c in MANY])
def test_topk_many_query_tokens(spd, name, B, T, lens, W, k):
    w = make_workload(name, B=B, T=T, seq_lens=lens, bt_width=W, k=k, seed=sum(map(ord, name)))
    sel, _ = _run(spd, w, k)
    for i in range(w.N):
        check_topk_row(sel[i], w, i, k)


def test_topk_four_tokens_all_equal_full_chunks(spd):
    """Four query tokens per request, every score of a row equal: 32-page
    chunks put 4096 tokens of each row in one histogram bin (the four-row
    scan packs two 16-bit counts per word), ties go to the lowest indices."""
    w = make_workload("eq4", B=64, T=4, seq_lens=32768, bt_width=256, k=1000, seed=16)
    codes = np.full((w.num_pages, 128, 128), 3, dtype=np.uint8)
    w.index_pool = mxfp4.pack(codes, np.full((w.num_pages, 128, 4), 127, dtype=np.uint8))
    sel, _ = _run(spd, w, 1000)
    ref = np.arange(1000)
    for i in range(w.N):
        assert np.array_equal(np.sort(sel[i]), ref), f"query {i}"


def test_topk_many_query_tokens_all_equal():
    """Every score equal in every row: the threshold bin overflows LDS, ties go to the lowest indices."""
    import sparse_paged_decode_amd as spd

    w = make_workload("eqmany", B=300, T=1, seq_lens=5000, bt_width=100, k=1000, seed=15)
    codes = np.full((w.num_pages, 128, 128), 3, dtype=np.uint8)
    w.index_pool = mxfp4.pack(codes, np.full((w.num_pages, 128, 4), 127, dtype=np.uint8))
    sel, _ = _run(spd, w, 1000)
    ref = np.arange(1000)
    for i in range(w.N):
        assert np.array_equal(np.sort(sel[i]), ref), f"query {i}"
