"""Indexer context parallelism, emulated on one device (CPU oracle, test infrastructure).

Source: page *vllm.models.minimax_m3.amd.mono.weights*, ``_build_cp_qkv``:
every rank keeps all G ranks' index-q heads, so that rank r can score its
own share of every sequence's index pages for all G heads; the per-head
candidates are then exchanged and each head's owner keeps its top-k.  The
pages print the weight gathering, not the exchange; the readings taken:

* Shard r of G owns the block-table columns [r * c, min(W, (r + 1) * c)),
  c = ceil(W / G), W the table width: a contiguous range of every
  sequence's pages (tokens [128 r c, 128 min(W, (r + 1) c))).
* Each shard emits, per head and query token, the top-k (score, position)
  pairs among its tokens that the query sees (positions 0..pos), with the
  same rule as the global selection: higher score first, ties to the lower
  position, NaN below every number; fewer than k tokens give all of them.
* The owner merges the G lists of a head by the same rule and keeps k.
  Every token of the global top-k is in its own shard's top-k, so the
  merged selection is the global one.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use this module.
"""

import numpy as np

from . import decode

PAGE_TOKENS = 128


def shard_windows(bt_width, G):
    """Page windows ``[(lo, hi), ...]`` of the G shards over a table of ``bt_width`` columns."""
    c = -(-int(bt_width) // int(G))
    return [(min(r * c, bt_width), min((r + 1) * c, bt_width)) for r in range(G)]


def _rank(scores, positions, k):
    """The top-k of (score, position) pairs: higher score, then lower position; NaN last."""
    order = np.lexsort((positions, -scores))
    take = order[: min(int(k), order.shape[0])]
    return positions[take], scores[take]


def shard_topk(index_q_bits, index_pool, bt_row, pos, k, window):
    """(positions, scores) of the top-k tokens of one shard window for one query at ``pos``."""
    lo, hi = window[0] * PAGE_TOKENS, window[1] * PAGE_TOKENS
    end = min(hi, int(pos) + 1)
    if end <= lo:
        return np.zeros(0, dtype=np.int64), np.zeros(0)
    s = decode.index_scores(index_q_bits, index_pool, bt_row, end - 1)
    positions = np.arange(lo, end, dtype=np.int64)
    return _rank(s[lo:end], positions, k)


def merge(candidates, k):
    """Top-k over the union of the shards' (positions, scores) lists."""
    if not candidates:
        return np.zeros(0, dtype=np.int64), np.zeros(0)
    positions = np.concatenate([c[0] for c in candidates])
    scores = np.concatenate([c[1] for c in candidates])
    return _rank(scores, positions, k)


def cp_index_topk(index_q_heads, index_pool, block_table, seq_lens, T, k, G):
    """Selections of every head and query token through G shards and a merge: int64 ``[H, B*T, k]``, -1 padded."""
    H, N = index_q_heads.shape[0], index_q_heads.shape[1]
    pos = decode.query_positions(seq_lens, T)
    windows = shard_windows(block_table.shape[1], G)
    out = np.full((H, N, k), -1, dtype=np.int64)
    for h in range(H):
        for i in range(N):
            bt_row = block_table[i // T]
            cands = [shard_topk(index_q_heads[h, i], index_pool, bt_row, pos[i], k, w) for w in windows]
            sel, _ = merge(cands, k)
            out[h, i, : sel.shape[0]] = sel
    return out
