"""GPU parity of the indexer context-parallel emulation (window scans + merge).

* A window call selects, per query token, the oracle's shard top-k (up to
  exact-tie order within the 1e-6 band of its k-th score) with absolute
  positions inside the window.
* The merge kernel reproduces the oracle's merge exactly (the same
  position and score pairs; the order within a row is free).
* Shards-then-merge (one C-ABI call: each shard scores its window for all
  heads in one launch, groups of up to four (head, token) rows sharing each
  page read) selects exactly the sets the global index call selects (same
  fp32 scores, same tie rule), and matches the oracle's global top-k.
"""

import numpy as np
import pytest
import torch

from helpers import bf16_tensor, check_topk_row, to_device
from oracle import cp, decode, mxfp4
from workloads import make_workload, workload

pytestmark = pytest.mark.gpu

TIE_BAND = 1e-6


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_amd as spd

    spd.load_library()
    assert torch.cuda.is_available()
    return spd


def _check_shard_row(sel_row, w, i, k, window):
    T = w.T
    b = i // T
    pos = int(w.seq_lens[b]) - T + i % T
    ref_p, ref_s = cp.shard_topk(w.index_q[i], w.index_pool, w.block_table[b], pos, k, window)
    n = ref_p.shape[0]
    got = np.asarray(sel_row)[:n]
    assert np.all(np.asarray(sel_row)[n:] == -1), f"query {i}: padding"
    lo, hi = window[0] * 128, min(window[1] * 128, pos + 1)
    assert np.all((got >= lo) & (got < hi)), f"query {i}: outside the window"
    assert np.unique(got).size == n
    if n == 0:
        return
    s = decode.index_scores(w.index_q[i], w.index_pool, w.block_table[b], pos)
    kth = ref_s[n - 1]
    diff = np.setxor1d(got, ref_p)
    assert np.all(np.abs(s[diff] - kth) <= TIE_BAND * abs(kth)), f"query {i}: differs beyond the tie band"


@pytest.mark.parametrize("T,lens,W,k,G", [(1, [1, 300, 1000, 2049], 17, 100, 4), (4, [4, 700, 3000], 24, 300, 3),
                                          (2, [5000, 260], 40, 2000, 2)], ids=["t1_g4", "t4_g3", "t2_g2_k_large"])
def test_window_calls_match_oracle_shards(spd, T, lens, W, k, G):
    w = make_workload(f"cpw{T}", B=len(lens), T=T, seq_lens=lens, bt_width=W, k=k, seed=70 + T, exp_range=(124, 127))
    d = to_device(w)
    for window in cp.shard_windows(W, G):
        print(f"[cp] window {window}", flush=True)
        sel, sc = spd.mono_index_score_topk(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], k, T=T,
                                            return_scores=True, page_window=window)
        torch.cuda.synchronize()
        sel = sel.cpu().numpy()
        for i in range(w.N):
            _check_shard_row(sel[i], w, i, k, window)


def test_merge_kernel_matches_oracle_exactly(spd):
    rng = np.random.default_rng(71)
    G, N, k_in, k = 3, 40, 50, 64
    idx = np.full((G, N, k_in), -1, dtype=np.int32)
    sc = np.full((G, N, k_in), np.nan, dtype=np.float32)
    for i in range(N):
        for g in range(G):
            n = int(rng.integers(0, k_in + 1))
            idx[g, i, :n] = g * 1000 + rng.permutation(1000)[:n]
            vals = rng.integers(1, 6, size=n).astype(np.float32) * rng.choice([-1, 1], size=n)  # many ties, no zeros
            vals[rng.random(n) < 0.05] = np.nan
            sc[g, i, :n] = vals
    out, out_s = spd.mono_topk_merge(torch.from_numpy(idx).cuda(), torch.from_numpy(sc).cuda(), k)
    torch.cuda.synchronize()
    out, out_s = out.cpu().numpy(), out_s.cpu().numpy()
    for i in range(N):
        lists = [(idx[g, i][idx[g, i] >= 0].astype(np.int64), sc[g, i][idx[g, i] >= 0].astype(np.float64))
                 for g in range(G)]
        want_p, want_s = cp.merge(lists, k)
        n = want_p.shape[0]
        # the same (position, score) pairs, in any order
        order = np.argsort(out[i, :n])
        want_order = np.argsort(want_p)
        np.testing.assert_array_equal(out[i, :n][order], want_p[want_order])
        np.testing.assert_array_equal(out_s[i, :n][order], want_s[want_order].astype(np.float32))
        assert np.all(out[i, n:] == -1) and np.all(np.isnan(out_s[i, n:]))


def _heads(w, H, seed):
    rng = np.random.default_rng(seed)
    extra = [mxfp4.round_to_bf16_bits(rng.standard_normal((w.N, 128))) for _ in range(H - 1)]
    return np.stack([w.index_q, *extra])


@pytest.mark.parametrize("H,G,T,lens,W,k", [(4, 4, 1, [1, 500, 3000, 9000], 71, 700), (2, 3, 4, [4, 1000, 2049], 17, 300),
                                            (3, 8, 1, [300, 600], 5, 100), (3, 2, 2, [2, 129, 4000], 33, 250),
                                            (5, 4, 3, [3, 777, 2500], 20, 64)],
                         ids=["h4_g4", "h2_g3_t4", "h3_g8_empty_shards", "h3_g2_t2_mixed_groups", "h5_g4_t3"])
def test_cp_equals_global_selection(spd, H, G, T, lens, W, k):
    w = make_workload(f"cp{H}{G}", B=len(lens), T=T, seq_lens=lens, bt_width=W, k=k, seed=72 + H, exp_range=(124, 127))
    d = to_device(w)
    heads = _heads(w, H, 73)
    got = spd.indexer_cp_topk(bf16_tensor(heads, "cuda"), d["index_pool"], d["block_table"], d["seq_lens"], k, T=T,
                              shards=G)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    for h in range(H):
        ref = spd.mono_index_score_topk(bf16_tensor(heads[h], "cuda"), d["index_pool"], d["block_table"],
                                        d["seq_lens"], k, T=T)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(np.sort(got[h], axis=1), np.sort(ref.cpu().numpy(), axis=1))
        wh = make_workload(f"cp{H}{G}", B=len(lens), T=T, seq_lens=lens, bt_width=W, k=k, seed=72 + H,
                           exp_range=(124, 127))
        wh.index_q = heads[h]
        for i in range(w.N):
            check_topk_row(got[h, i], wh, i, k)


def test_cp_full_size(spd):
    """64 requests of 32768 tokens, top-2048, 4 index heads over 4 shards."""
    w = workload(3)
    d = to_device(w)
    heads = _heads(w, 4, 74)
    print("[cp] full size", flush=True)
    got = spd.indexer_cp_topk(bf16_tensor(heads, "cuda"), d["index_pool"], d["block_table"], d["seq_lens"], w.k,
                              shards=4)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    for h in range(4):
        ref = spd.mono_index_score_topk(bf16_tensor(heads[h], "cuda"), d["index_pool"], d["block_table"],
                                        d["seq_lens"], w.k)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(np.sort(got[h], axis=1), np.sort(ref.cpu().numpy(), axis=1))
    w.index_q = heads[2]
    for i in (0, 40):
        check_topk_row(got[2, i], w, i, w.k)


def test_merge_all_ties_and_full_lists(spd):
    # 4 full lists of 2048 equal scores: the k lowest positions win.
    G, N, k_in, k = 4, 3, 2048, 2048
    rng = np.random.default_rng(75)
    idx = np.stack([np.stack([g * 100000 + rng.permutation(100000)[:k_in] for _ in range(N)]) for g in range(G)])
    idx = idx.astype(np.int32)
    sc = np.ones((G, N, k_in), dtype=np.float32)
    out, out_s = spd.mono_topk_merge(torch.from_numpy(idx).cuda(), torch.from_numpy(sc).cuda(), k)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for i in range(N):
        want = np.sort(idx[:, i].ravel())[:k]
        np.testing.assert_array_equal(np.sort(out[i]), want)
    assert np.all(out_s.cpu().numpy() == 1.0)
