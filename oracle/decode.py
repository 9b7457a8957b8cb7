"""Index scoring, top-k selection and paged GQA decode attention (CPU oracle).

Test infrastructure: only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may use this module.

Sources and readings (each function repeats the one it relies on):

* Token addressing.  Page *vllm.models.minimax_m3.amd.mono.dispatch*,
  ``_step_refusal`` and ``_slots_shared``: one int32 block table, rows
  ``bt_width`` apart, shared by K, V and the index key, and int32 seq_lens.
  Reading: logical token j of request b lives in physical page
  ``block_table[b, j // 128]``, row ``j % 128`` (the page-128 convention of
  the mxfp4_pages page).
* Multi-token decode.  Same page, ``_step_refusal``: a step decodes ``q``
  tokens per request, ``n = batch * q`` in all, flattened request-major.
  Reading: ``seq_lens`` counts every token including the ``T`` being
  decoded, so query t of request b sits at position ``L_b - T + t`` and sees
  tokens ``0 .. L_b - T + t`` (causal).
* Index scores.  The mxfp4_pages page names the index scorers without giving
  their rule.  Reading: the score of token j is the dot product of the
  dequantised bf16 index-q row with the dequantised index-K row j; no ReLU,
  weights, scale or bias.  Here it is exact (float64 over exact products).
* Top-k.  Per query token, the k highest-scoring valid tokens; ties go to
  the lower token index; with fewer than k valid tokens, all of them.  A NaN
  score ranks below every number.
* Cache formats.  MXFP4 pages (8704 B, ``oracle.mxfp4``) or the older
  build's fp8 pages (16384 B, ``oracle.fp8``), told apart by the page size;
  with fp8, K and V values carry the per-tensor ``k_scale`` / ``v_scale``.
* Attention.  Per query token: ``z_hj = scale * q_h . k_j`` over the
  candidate tokens (the selected ones, or every valid one when there is no
  selection), ``p = softmax_j(z)`` and ``o_h = sum_j p_hj v_j``.  All 16
  query heads read the one KV head.  No sink, soft-cap, ALiBi or window.
  An empty candidate set gives a zero output.

All arithmetic is float64.
"""

import numpy as np

from . import fp8, mxfp4

Q_HEADS = 16  # query heads per KV head
HEAD_DIM = 128


def query_positions(seq_lens, T):
    """Position of every query token, flattened request-major (i = b*T + t).

    Query t of request b is at ``seq_lens[b] - T + t`` (the T decoded tokens
    are the last T of the sequence).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    t = np.arange(T, dtype=np.int64)
    return (seq_lens[:, None] - T + t[None, :]).reshape(-1)


def sequence_rows(pool, bt_row, n_tokens, head=None):
    """Exact dequantised rows ``[n_tokens, 128]`` of tokens 0..n_tokens-1.

    ``pool`` is ``[P, page]`` (index key) or ``[P, H, page]`` with ``head``
    picking the KV head; a page of 8704 bytes is MXFP4, of 16384 bytes fp8
    (without its tensor scale).  Token j comes from page ``bt_row[j // 128]``,
    row ``j % 128``.
    """
    if n_tokens <= 0:
        return np.zeros((0, HEAD_DIM))
    page_bytes = pool.shape[-1]
    if page_bytes == mxfp4.PAGE_BYTES:
        dequant = mxfp4.dequant
    elif page_bytes == fp8.PAGE_BYTES:
        dequant = fp8.dequant
    else:
        raise ValueError(f"unknown page size {page_bytes}")
    n_pages = -(-n_tokens // mxfp4.PAGE_TOKENS)
    page_ids = np.asarray(bt_row[:n_pages], dtype=np.int64)
    pages = pool[page_ids] if head is None else pool[page_ids, head]
    rows = dequant(pages).reshape(n_pages * mxfp4.PAGE_TOKENS, HEAD_DIM)
    return rows[:n_tokens]


def scores_of_rows(index_q_bits, rows):
    """Exact scores of dequantised index-key rows ``[n, 128]`` for one query token.

    ``index_q_bits``: bf16 bit patterns ``[128]``.  The score of a row is its
    dot product with the dequantised index-q row (float64; every product of a
    bf16 value and an MXFP4 or e4m3 value is exact).
    """
    return rows @ mxfp4.bf16_bits_to_f64(index_q_bits)


def index_scores(index_q_bits, index_pool, bt_row, pos):
    """Exact scores ``s[j]`` of tokens ``j = 0..pos`` for one query token.

    ``index_q_bits``: bf16 bit patterns ``[128]``.  The score is the dot
    product of the dequantised index-q row with each dequantised index-K row.
    """
    return scores_of_rows(index_q_bits, sequence_rows(index_pool, bt_row, int(pos) + 1))


def topk(scores, k):
    """Token indices of the top ``min(k, len(scores))`` scores.

    Full stable sort by (descending score, ascending index): ties go to the
    lower index and NaN ranks last.
    """
    scores = np.asarray(scores, dtype=np.float64)
    idx = np.arange(scores.shape[0])
    order = np.lexsort((idx, -scores))
    return order[: min(int(k), scores.shape[0])]


def index_topk(index_q_bits, index_pool, block_table, seq_lens, T, k):
    """Selections for every query token: int64 ``[B*T, k]`` padded with -1."""
    pos = query_positions(seq_lens, T)
    out = np.full((pos.shape[0], k), -1, dtype=np.int64)
    for i, p in enumerate(pos):
        s = index_scores(index_q_bits[i], index_pool, block_table[i // T], p)
        sel = topk(s, k)
        out[i, : sel.shape[0]] = sel
    return out


def candidates(pos, selected_row=None):
    """Candidate tokens of one query token at position ``pos``.

    Without a selection: every valid token ``0..pos``.  With one: the listed
    entries that are valid, in list order (entries < 0 or > pos are dropped).
    """
    if selected_row is None:
        return np.arange(int(pos) + 1, dtype=np.int64)
    sel = np.asarray(selected_row, dtype=np.int64)
    return sel[(sel >= 0) & (sel <= pos)]


def softmax_weights(q_bits, k_rows, scale):
    """Softmax weights ``p [16, n]`` of 16 query heads over K rows ``[n, 128]``
    (float64): ``p_hj = exp(z_hj - max_j z_hj) / sum_j exp(...)`` with
    ``z_hj = scale * q_h . k_j``."""
    q = mxfp4.bf16_bits_to_f64(q_bits)
    z = scale * (q @ k_rows.T)  # [16, n]
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=1, keepdims=True)


def attend(q_bits, k_rows, v_rows, scale):
    """Softmax attention of 16 query heads over gathered K/V rows (float64).

    ``q_bits`` bf16 bits ``[16, 128]``; ``k_rows``/``v_rows`` ``[n, 128]``.
    Returns ``[16, 128]``; zeros when n == 0.
    """
    if k_rows.shape[0] == 0:
        return np.zeros((np.asarray(q_bits).shape[0], HEAD_DIM))
    return softmax_weights(q_bits, k_rows, scale) @ v_rows


def decode_rows(q_bits, k_rows, v_rows, pos, scale, selected_row=None, k_scale=1.0, v_scale=1.0):
    """Attention output ``[16, 128]`` for one query token from its request's rows.

    ``k_rows`` / ``v_rows``: the request's dequantised K and V rows of tokens
    ``0..n-1`` (``sequence_rows``), with n past every candidate.  ``k_scale``
    / ``v_scale`` multiply every K / V value (the fp8 caches' per-tensor
    scales; 1 for MXFP4); the products are exact in float64.
    """
    cand = candidates(pos, selected_row)
    return attend(q_bits, k_rows[cand] * float(k_scale), v_rows[cand] * float(v_scale), scale)


def decode_one(q_bits, k_pool, v_pool, bt_row, pos, scale, selected_row=None, head=0, k_scale=1.0, v_scale=1.0):
    """Attention output ``[16, 128]`` for one query token.

    ``k_scale`` / ``v_scale`` multiply every K / V value (the fp8 caches'
    per-tensor scales; 1 for MXFP4).  The products are exact in float64.
    """
    cand = candidates(pos, selected_row)
    n_seen = int(cand.max()) + 1 if cand.size else 0
    k_all = sequence_rows(k_pool, bt_row, n_seen, head)
    v_all = sequence_rows(v_pool, bt_row, n_seen, head)
    return decode_rows(q_bits, k_all, v_all, pos, scale, selected_row, k_scale, v_scale)


def pa_decode(q_bits, k_pool, v_pool, block_table, seq_lens, T, scale, selected=None, head=0, k_scale=1.0,
              v_scale=1.0):
    """Attention for every query token: float64 ``[B*T, 16, 128]``."""
    pos = query_positions(seq_lens, T)
    out = np.zeros((pos.shape[0], q_bits.shape[1], HEAD_DIM))
    for i, p in enumerate(pos):
        row = None if selected is None else selected[i]
        out[i] = decode_one(q_bits[i], k_pool, v_pool, block_table[i // T], p, scale, row, head, k_scale, v_scale)
    return out
