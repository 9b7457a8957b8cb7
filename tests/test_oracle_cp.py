"""Pins of the oracle's indexer context-parallel emulation.

The shards-then-merge selection must equal the global top-k (every token of
the global top-k is in its shard's top-k): checked against the pinned
``decode.index_topk`` on ragged, tie-heavy and multi-token cases, against a
brute-force rank count on tiny inputs, and on the window geometry itself.
"""

import numpy as np
import pytest

from oracle import cp, decode, mxfp4
from workloads import make_workload


def test_shard_windows_cover_the_table_once():
    for W in (1, 2, 7, 64, 257):
        for G in (1, 2, 3, 4, 8):
            wins = cp.shard_windows(W, G)
            assert len(wins) == G
            covered = np.concatenate([np.arange(lo, hi) for lo, hi in wins])
            np.testing.assert_array_equal(covered, np.arange(W))
            assert all(lo <= hi for lo, hi in wins)


@pytest.mark.parametrize("G", [1, 2, 3, 4])
@pytest.mark.parametrize("T,lens,k", [(1, [1, 130, 700], 50), (4, [4, 300, 1000], 37), (2, [600, 129], 1000)])
def test_cp_equals_global_topk(G, T, lens, k):
    w = make_workload("cp", B=len(lens), T=T, seq_lens=lens, bt_width=8, k=k, seed=61 + G, exp_range=(124, 127))
    rng = np.random.default_rng(62)
    heads = np.stack([w.index_q, mxfp4.round_to_bf16_bits(rng.standard_normal((w.N, 128)))])
    got = cp.cp_index_topk(heads, w.index_pool, w.block_table, w.seq_lens, T, k, G)
    for h in range(2):
        want = decode.index_topk(heads[h], w.index_pool, w.block_table, w.seq_lens, T, k)
        np.testing.assert_array_equal(got[h], want)


def test_cp_ties_go_to_the_lowest_positions():
    # Every index row is identical: all scores tie, so the selection is the
    # k lowest positions, whichever shards they come from.
    w = make_workload("cp_ties", B=1, T=1, seq_lens=[900], bt_width=8, k=300, seed=63)
    w.index_pool[:] = w.index_pool[0]
    row = w.index_pool[0].copy()
    pages = np.repeat(row[None], w.index_pool.shape[0], axis=0)
    data, scale = mxfp4.page_views(pages)
    data[:] = data[:, :1]
    scale[:] = scale[:, :1]
    got = cp.cp_index_topk(w.index_q[None], pages, w.block_table, w.seq_lens, 1, 300, 4)
    np.testing.assert_array_equal(got[0, 0], np.arange(300))


def test_merge_brute_force_small():
    rng = np.random.default_rng(64)
    for _ in range(200):
        n_lists = rng.integers(1, 4)
        lists, all_p, all_s = [], [], []
        base = 0
        for _ in range(n_lists):
            n = rng.integers(0, 6)
            p = base + rng.permutation(10)[:n]
            base += 10
            s = rng.integers(-2, 3, size=n).astype(float)  # many ties
            s[rng.random(n) < 0.1] = np.nan
            lists.append((p, s))
            all_p.append(p)
            all_s.append(s)
        k = int(rng.integers(1, 8))
        got, _ = cp.merge(lists, k)
        p = np.concatenate(all_p)
        s = np.concatenate(all_s)
        # rank of each pair = number of pairs strictly before it
        def before(a, b):  # pair a ranks before pair b
            sa, sb = s[a], s[b]
            if np.isnan(sa) and np.isnan(sb):
                return p[a] < p[b]
            if np.isnan(sb):
                return True
            if np.isnan(sa):
                return False
            return sa > sb or (sa == sb and p[a] < p[b])
        ranks = [sum(before(b, a) for b in range(len(p))) for a in range(len(p))]
        want = [p[a] for a in sorted(range(len(p)), key=lambda a: ranks[a])][:k]
        np.testing.assert_array_equal(got, want)
