"""Pins of the oracle's positions, index scores, top-k and attention.

The checks come from outside the oracle: closed forms on constructed pages,
brute-force rank counting, torch.topk, torch's fp64 scaled-dot-product
attention on gathered rows, and invariances the mathematics fixes.
"""

import itertools

import numpy as np
import pytest
import torch

from oracle import decode, mxfp4
from workloads import make_workload


def _bits_to_f64_torch(bits):
    return torch.from_numpy(np.asarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _one_hot_pool(n_pages, dims, code=2, exp=127):
    """Index-K pool where row j (flat over pages) has one nonzero element at dims[j]."""
    codes = np.zeros((n_pages, 128, 128), dtype=np.uint8)
    flat = codes.reshape(n_pages * 128, 128)
    flat[np.arange(n_pages * 128), dims] = code
    scales = np.full((n_pages, 128, 4), exp, dtype=np.uint8)
    return mxfp4.pack(codes, scales)


# --- positions ------------------------------------------------------------------


def test_query_positions_closed_form():
    np.testing.assert_array_equal(decode.query_positions([5, 9], 1), [4, 8])
    # multi-token decode: the last T tokens, positions L-4..L-1
    np.testing.assert_array_equal(decode.query_positions([10, 300], 4), [6, 7, 8, 9, 296, 297, 298, 299])


# --- index scores ---------------------------------------------------------------


def test_index_scores_one_hot_closed_form():
    """Row j holds 1.0 at dim d_j only, so s[j] = iq[d_j] through a permuted table."""
    rng = np.random.default_rng(3)
    n_pages = 4
    dims = (np.arange(n_pages * 128) * 37 + 5) % 128
    phys = _one_hot_pool(n_pages, dims)  # physical page p, row r <-> flat row p*128 + r
    perm = np.array([2, 0, 3, 1])
    bt_row = perm  # logical page lp -> physical page perm[lp]
    iq_bits = mxfp4.round_to_bf16_bits(rng.standard_normal(128))
    iq = _bits_to_f64_torch(iq_bits)
    pos = 3 * 128 + 40  # partial last page
    s = decode.index_scores(iq_bits, phys, bt_row, pos)
    assert s.shape == (pos + 1,)
    j = np.arange(pos + 1)
    phys_row = perm[j // 128] * 128 + j % 128
    np.testing.assert_array_equal(s, iq[dims[phys_row]])


def test_index_scores_scale_and_sign():
    """code 15 (-6.0) with e = 130 (x8) gives -48 * iq[d]."""
    dims = np.full(128, 9)
    pool = _one_hot_pool(1, dims, code=15, exp=130)
    iq_bits = mxfp4.round_to_bf16_bits(np.linspace(-1, 1, 128))
    iq = _bits_to_f64_torch(iq_bits)
    s = decode.index_scores(iq_bits, pool, [0], 127)
    np.testing.assert_array_equal(s, np.full(128, -48.0 * iq[9]))


def test_index_scores_against_torch_matmul():
    w = make_workload("t", B=2, T=2, seq_lens=[300, 129], bt_width=3, k=16, seed=5)
    pos = decode.query_positions(w.seq_lens, w.T)
    pool_t = torch.from_numpy(w.index_pool)
    for i, p in enumerate(pos):
        b = i // w.T
        # gather through torch: pages by block table, then flatten and cut
        pg = torch.from_numpy(w.block_table[b, : (p // 128) + 1].astype(np.int64))
        rows = pool_t.index_select(0, pg)
        data = rows[:, :8192].reshape(-1, 128, 64).to(torch.int64)
        nib = torch.stack([data % 16, data // 16], dim=-1).reshape(-1, 128, 128)
        table = torch.tensor([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6], dtype=torch.float64)
        sc = rows[:, 8192:].reshape(-1, 128, 4).contiguous().view(torch.float8_e8m0fnu).to(torch.float64)
        x = (table[nib] * sc.repeat_interleave(32, dim=-1)).reshape(-1, 128)[: p + 1]
        iq = torch.from_numpy(w.index_q[i].view(np.int16)).view(torch.bfloat16).to(torch.float64)
        ref = torch.matmul(x, iq).numpy()
        s = decode.index_scores(w.index_q[i], w.index_pool, w.block_table[b], p)
        np.testing.assert_allclose(s, ref, rtol=1e-13, atol=0)


# --- top-k ----------------------------------------------------------------------


def _rank_select(scores, k):
    """Brute force: j is selected iff fewer than k tokens beat it (higher score, or equal and lower index)."""
    n = len(scores)
    sel = []
    for j in range(n):
        better = sum(1 for i in range(n) if scores[i] > scores[j] or (scores[i] == scores[j] and i < j))
        if better < k:
            sel.append(j)
    return sorted(sel)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(9)
    for trial in range(200):
        n = int(rng.integers(1, 12))
        s = rng.integers(-3, 4, size=n).astype(np.float64)  # many ties
        k = int(rng.integers(1, 14))
        got = sorted(decode.topk(s, k).tolist())
        assert got == _rank_select(s, k), (s, k)


def test_topk_special_cases():
    s = np.array([0.5, 2.0, -1.0, 2.0, 1.5])
    assert decode.topk(s, 1).tolist() == [1]  # argmax, lower index on a tie
    assert decode.topk(s, 1).tolist() == [int(np.argmax(s))]
    assert sorted(decode.topk(s, 5).tolist()) == [0, 1, 2, 3, 4]
    assert sorted(decode.topk(s, 99).tolist()) == [0, 1, 2, 3, 4]
    rng = np.random.default_rng(1)
    d = rng.standard_normal(1000)
    ref = torch.topk(torch.from_numpy(d), 37).indices.numpy()
    assert set(decode.topk(d, 37).tolist()) == set(ref.tolist())
    # NaN ranks last
    assert decode.topk(np.array([np.nan, -5.0, 1.0]), 2).tolist() == [2, 1]


def test_index_topk_shapes_and_padding():
    w = make_workload("t", B=3, T=2, seq_lens=[2, 200, 131], bt_width=2, k=40, seed=2)
    sel = decode.index_topk(w.index_q, w.index_pool, w.block_table, w.seq_lens, w.T, w.k)
    pos = decode.query_positions(w.seq_lens, w.T)
    assert sel.shape == (6, 40)
    for i, p in enumerate(pos):
        valid = sel[i][sel[i] >= 0]
        assert len(valid) == min(40, p + 1)
        assert len(set(valid.tolist())) == len(valid) and valid.max() <= p
        assert np.all(sel[i][len(valid) :] == -1)


# --- attention ------------------------------------------------------------------


def _sdpa(q_bits, k_rows, v_rows, scale):
    q = torch.from_numpy(_bits_to_f64_torch(q_bits))[None, :, None, :]  # [1,16,1,128]
    k = torch.from_numpy(k_rows)[None, None].expand(1, 16, -1, -1).contiguous()
    v = torch.from_numpy(v_rows)[None, None].expand(1, 16, -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    return o[0, :, 0, :].numpy()


def _small(seq_len, seed, **kw):
    return make_workload("t", B=1, T=1, seq_lens=seq_len, bt_width=2, k=0, seed=seed, **kw)


@pytest.mark.parametrize("seq_len", [1, 77, 128, 200, 256])
def test_attention_against_torch_sdpa(seq_len):
    for exps in [(122, 132), (124, 124), (127, 127)]:
        w = _small(seq_len, seed=seq_len, exp_range=exps)
        o = decode.pa_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, 1, w.scale)[0]
        # independent gather: page-major flatten through the block table
        kk = mxfp4.dequant(w.k_pool[:, 0])[w.block_table[0, : -(-seq_len // 128)]].reshape(-1, 128)[:seq_len]
        vv = mxfp4.dequant(w.v_pool[:, 0])[w.block_table[0, : -(-seq_len // 128)]].reshape(-1, 128)[:seq_len]
        ref = _sdpa(w.q[0], kk, vv, w.scale)
        np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12 * np.abs(vv).max())


def _pages_from(codes_fn, exps, n_pages):
    codes = np.fromfunction(codes_fn, (n_pages, 128, 128), dtype=np.int64).astype(np.uint8) & 0xF
    return mxfp4.pack(codes, np.full((n_pages, 128, 4), exps, dtype=np.uint8))[:, None, :]


def test_attention_closed_forms():
    w = _small(200, seed=4, exp_range=(124, 130))
    bt, L = w.block_table[0], 200
    V = decode.sequence_rows(w.v_pool, bt, L, 0)
    # q = 0 -> mean of V over the candidates
    zq = np.zeros_like(w.q[0])
    o = decode.decode_one(zq, w.k_pool, w.v_pool, bt, L - 1, w.scale)
    np.testing.assert_allclose(o, np.broadcast_to(V.mean(0), (16, 128)), rtol=1e-12, atol=1e-12)
    # one valid token -> V_0
    o1 = decode.decode_one(w.q[0], w.k_pool, w.v_pool, bt, 0, w.scale)
    np.testing.assert_array_equal(o1, np.broadcast_to(V[0], (16, 128)))
    # all K rows equal -> mean of V
    kpool = _pages_from(lambda p, r, i: i % 16, 126, 2)
    o2 = decode.decode_one(w.q[0], kpool, w.v_pool, bt, L - 1, w.scale)
    np.testing.assert_allclose(o2, np.broadcast_to(V.mean(0), (16, 128)), rtol=1e-12, atol=1e-12)
    # constant V -> that constant (code 5 = 3.0, e = 126 -> 1.5)
    vpool = _pages_from(lambda p, r, i: 0 * i + 5, 126, 2)
    o3 = decode.decode_one(w.q[0], w.k_pool, vpool, bt, L - 1, w.scale)
    np.testing.assert_allclose(o3, 1.5, rtol=1e-14)
    # selection: only the listed valid tokens count, -1 and > pos dropped
    sel = np.array([5, -1, 150, 199, 3000])
    o4 = decode.decode_one(w.q[0], w.k_pool, w.v_pool, bt, 160, w.scale, sel)
    K = decode.sequence_rows(w.k_pool, bt, L, 0)
    ref = _sdpa(w.q[0], K[[5, 150]], V[[5, 150]], w.scale)
    np.testing.assert_allclose(o4, ref, rtol=1e-10, atol=1e-12)
    # empty candidate set -> zeros
    o5 = decode.decode_one(w.q[0], w.k_pool, w.v_pool, bt, 10, w.scale, np.array([-1, 50]))
    np.testing.assert_array_equal(o5, 0.0)


def test_attention_invariances():
    w = make_workload("t", B=2, T=2, seq_lens=[250, 140], bt_width=2, k=0, seed=8, exp_range=(124, 127))
    base = decode.pa_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, 2, w.scale)
    # pool-page permutation with a matching block-table relabel
    P = w.num_pages
    perm = np.random.default_rng(0).permutation(P)
    inv = np.argsort(perm)
    bt2 = np.where(w.block_table >= 0, inv[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    o = decode.pa_decode(w.q, w.k_pool[perm], w.v_pool[perm], bt2, w.seq_lens, 2, w.scale)
    np.testing.assert_array_equal(o, base)
    # sparse with every valid token selected equals dense
    pos = decode.query_positions(w.seq_lens, 2)
    sel = np.full((4, 256), -1)
    for i, p in enumerate(pos):
        sel[i, : p + 1] = np.random.default_rng(i).permutation(p + 1)
    o = decode.pa_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, 2, w.scale, sel)
    np.testing.assert_allclose(o, base, rtol=1e-12, atol=1e-13)
    # K exponents + 1 with scale / 2: identical logits
    k2 = w.k_pool.copy()
    k2[..., 8192:] += 1
    o = decode.pa_decode(w.q, k2, w.v_pool, w.block_table, w.seq_lens, 2, w.scale / 2)
    np.testing.assert_array_equal(o, base)
    # V exponents + 1: output doubles
    v2 = w.v_pool.copy()
    v2[..., 8192:] += 1
    o = decode.pa_decode(w.q, w.k_pool, v2, w.block_table, w.seq_lens, 2, w.scale)
    np.testing.assert_allclose(o, 2 * base, rtol=1e-14, atol=0)


def test_multi_token_causality():
    """Query t sees tokens 0..L-T+t: changing token L-1 moves only the last query."""
    w = make_workload("t", B=1, T=4, seq_lens=[300], bt_width=3, k=0, seed=12, exp_range=(124, 124))
    base = decode.pa_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, 4, w.scale)
    v2 = w.v_pool.copy()
    last_page = w.block_table[0, 299 // 128]
    v2[last_page, 0, (299 % 128) * 64 : (299 % 128) * 64 + 64] ^= 0x11
    o = decode.pa_decode(w.q, w.k_pool, v2, w.block_table, w.seq_lens, 4, w.scale)
    np.testing.assert_array_equal(o[:3], base[:3])
    assert not np.array_equal(o[3], base[3])


def test_brute_force_tiny_sparse_step():
    """Tiny end-to-end: top-k by brute-force ranking then attention by SDPA."""
    w = make_workload("t", B=1, T=1, seq_lens=[60], bt_width=1, k=7, seed=21, exp_range=(125, 128))
    sel = decode.index_topk(w.index_q, w.index_pool, w.block_table, w.seq_lens, 1, w.k)[0]
    ik = mxfp4.dequant(w.index_pool[w.block_table[0, 0]])[:60]
    iq = _bits_to_f64_torch(w.index_q[0])
    scores = [float(sum(ik[j, d] * iq[d] for d in range(128))) for j in range(60)]
    assert sorted(sel.tolist()) == _rank_select(scores, 7)
    best = max(itertools.combinations(range(60), 1), key=lambda c: scores[c[0]])
    assert best[0] in sel.tolist()
    K = mxfp4.dequant(w.k_pool[w.block_table[0, 0], 0])[:60]
    V = mxfp4.dequant(w.v_pool[w.block_table[0, 0], 0])[:60]
    o = decode.pa_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, 1, w.scale, sel[None])[0]
    np.testing.assert_allclose(o, _sdpa(w.q[0], K[sel], V[sel], w.scale), rtol=1e-10, atol=1e-12)
