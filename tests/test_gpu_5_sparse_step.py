"""GPU parity of the one-launch sparse decode step (index top-k, then
attention over the selection) against the oracle.

The selection is checked as the index call's is (the oracle's top-k up to
exact-tie order, within a 1e-6 relative band of the k-th score); the output
is checked against the oracle's attention over the selection the call
returned, to the attention tolerance (relative L2 <= 5e-3, max |err| <=
1e-2 max|V|).
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


def _step(spd, w, d, ws):
    out, sel = spd.mono_sparse_decode_mxfp4(d["index_q"], d["index_pool"], d["q"], d["k_pool"], d["v_pool"],
                                            d["block_table"], d["seq_lens"], w.k, w.scale, T=w.T, workspace=ws)
    torch.cuda.synchronize()
    return out, sel


def _check_token(w, i, sel_row, out_bits):
    b = i // w.T
    pos = int(w.seq_lens[b]) - w.T + i % w.T
    check_topk_row(sel_row, w, i, w.k)
    ref = decode.decode_one(w.q[i], w.k_pool, w.v_pool, w.block_table[b], pos, w.scale, sel_row)
    vmax = float(np.abs(decode.sequence_rows(w.v_pool, w.block_table[b], pos + 1, 0)).max())
    o = mxfp4.bf16_bits_to_f64(out_bits[i])
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(o - ref) / nref if nref > 0 else np.linalg.norm(o)
    assert rel <= 5e-3 and np.max(np.abs(o - ref)) <= 1e-2 * vmax, (i, rel)


SMALL = [
    # name, B, T, seq_lens, bt_width, k, exps
    ("one_page", 1, 1, [100], 1, 10, (124, 127)),
    ("k_ge_valid", 2, 1, [50, 129], 2, 200, (122, 132)),
    ("k_one", 3, 1, [1, 128, 700], 6, 1, (124, 127)),
    ("ragged_multi_token", 4, 4, [4, 300, 1000, 2049], 17, 37, (124, 127)),
    ("several_chunks", 2, 1, [5000, 4097], 40, 700, (122, 132)),
    ("several_slices", 2, 1, [9000, 12289], 97, 300, (124, 126)),
    ("t3_group", 2, 3, [640, 3001], 24, 250, (124, 127)),
    ("t6_two_groups", 2, 6, [900, 2300], 18, 128, (122, 132)),
    # score rows longer than 64K: the slice-and-resolve selection
    ("wide_table_slices", 2, 1, [3000, 9000], 520, 700, (124, 127)),
    ("wide_table_slices_t3", 2, 3, [5000, 9100], 520, 300, (122, 132)),
]


@pytest.mark.parametrize("name,B,T,lens,W,k,exps", SMALL, ids=[c[0] for c in SMALL])
def test_step_small(spd, name, B, T, lens, W, k, exps):
    w = make_workload(name, B=B, T=T, seq_lens=lens, bt_width=W, k=k, seed=sum(map(ord, name)) + 7,
                      exp_range=exps)
    d = to_device(w)
    ws = spd.Workspace("cuda")
    out, sel = _step(spd, w, d, ws)
    assert spd.check_device_errors(ws) == 0
    sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
    for i in range(w.N):
        _check_token(w, i, sel_np[i], out_bits)
    # The same selection as the index call (as sets), and the workspace
    # serves the next call: the queue and every counter were reset.
    sel2 = spd.mono_index_score_topk(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], w.k, T=w.T)
    np.testing.assert_array_equal(np.sort(sel2.cpu().numpy(), axis=1), np.sort(sel_np, axis=1))
    out3, sel3 = _step(spd, w, d, ws)
    np.testing.assert_array_equal(np.sort(sel3.cpu().numpy(), axis=1), np.sort(sel_np, axis=1))
    a = mxfp4.bf16_bits_to_f64(bf16_bits(out3))
    b = mxfp4.bf16_bits_to_f64(out_bits)
    assert np.max(np.abs(a - b)) <= 1e-2 * max(np.max(np.abs(b)), 1e-30)


def test_step_equals_two_calls(spd):
    """Fused output matches the index call followed by the attention call."""
    w = make_workload("two", B=3, T=2, seq_lens=[3000, 5000, 4100], bt_width=40, k=512, seed=8,
                      exp_range=(124, 126))
    d = to_device(w)
    out, sel = _step(spd, w, d, spd.Workspace("cuda"))
    sel2 = spd.mono_index_score_topk(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], w.k, T=w.T)
    out2 = spd.mono_pa_decode_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], sel2,
                                    w.scale, T=w.T)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np.sort(sel2.cpu().numpy(), axis=1), np.sort(sel.cpu().numpy(), axis=1))
    a = mxfp4.bf16_bits_to_f64(bf16_bits(out))
    b = mxfp4.bf16_bits_to_f64(bf16_bits(out2))
    # same tokens in another order: equal up to fp32 summation order
    assert np.max(np.abs(a - b)) <= 1e-2 * np.max(np.abs(b))


def test_step_bad_page_id_is_flagged(spd):
    w = make_workload("badstep", B=2, T=1, seq_lens=[300, 300], bt_width=3, k=16, seed=9)
    d = to_device(w)
    d["block_table"][1, 1] = 10**6
    ws = spd.Workspace("cuda")
    _step(spd, w, d, ws)
    assert spd.check_device_errors(ws) & spd.DEVERR_PAGE_ID


def test_step_bad_seq_len_is_flagged_and_others_complete(spd):
    """A request whose length exceeds its block-table row is skipped and
    flagged; the other requests are still decoded."""
    w = make_workload("badlen", B=2, T=1, seq_lens=[300, 200], bt_width=3, k=64, seed=10, exp_range=(124, 127))
    d = to_device(w)
    d["seq_lens"][1] = 3 * 128 + 1
    ws = spd.Workspace("cuda")
    out, sel = _step(spd, w, d, ws)
    assert spd.check_device_errors(ws) & spd.DEVERR_SEQ_LEN
    _check_token(w, 0, sel.cpu().numpy()[0], bf16_bits(out))
    # the workspace is usable again after the flagged call
    d["seq_lens"][1] = 200
    out, sel = _step(spd, w, d, ws)
    assert spd.check_device_errors(ws) == 0
    sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
    for i in range(2):
        _check_token(w, i, sel_np[i], out_bits)


def test_one_workspace_across_shapes_and_entry_points(spd):
    """One buffer for every call, shapes growing and shrinking: each call
    clears what the previous ones left in its zero region."""
    ws = spd.Workspace("cuda", 64 << 20)
    shapes = [
        dict(B=1, T=1, seq_lens=[700], bt_width=6, k=64),
        dict(B=3, T=4, seq_lens=[300, 5000, 2100], bt_width=40, k=256),
        dict(B=2, T=1, seq_lens=[9000, 129], bt_width=71, k=100),
        dict(B=1, T=2, seq_lens=[400], bt_width=4, k=32),
    ]
    for n, kw in enumerate(shapes):
        w = make_workload(f"ws{n}", seed=100 + n, exp_range=(124, 127), **kw)
        d = to_device(w)
        sel_i = spd.mono_index_score_topk(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], w.k, T=w.T,
                                          workspace=ws)
        out_d = spd.mono_pa_decode_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], None,
                                         w.scale, T=w.T, workspace=ws)
        out, sel = _step(spd, w, d, ws)
        assert spd.check_device_errors(ws) == 0
        sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
        np.testing.assert_array_equal(np.sort(sel_i.cpu().numpy(), axis=1), np.sort(sel_np, axis=1))
        for i in range(w.N):
            _check_token(w, i, sel_np[i], out_bits)
        ref = decode.pa_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens, w.T, w.scale, None)
        o = mxfp4.bf16_bits_to_f64(bf16_bits(out_d))
        assert np.linalg.norm(o - ref) <= 5e-3 * np.linalg.norm(ref), f"dense attention, shape {n}"


def test_step_many_query_tokens(spd):
    """More filter slices than two rounds of the resident workgroups: one
    workgroup selects each token, inline in the last scan chunk (T = 1) or
    as a published item (T = 2)."""
    for name, B, T in (("many_step_t1", 300, 1), ("many_step_t2", 150, 2)):
        w = make_workload(name, B=B, T=T, seq_lens=(100, 3000), bt_width=100, k=300, seed=sum(map(ord, name)),
                          exp_range=(124, 127))
        d = to_device(w)
        ws = spd.Workspace("cuda")
        out, sel = _step(spd, w, d, ws)
        assert spd.check_device_errors(ws) == 0
        sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
        for i in range(0, w.N, 7):
            _check_token(w, i, sel_np[i], out_bits)
        for i in range(w.N):
            check_topk_row(sel_np[i], w, i, w.k)


def test_step_multiple_kv_heads(spd):
    """Three KV heads (48 query heads), several attention splits per head and
    two query tokens per request: every head against the oracle with the
    selection the call returned (the heads share it)."""
    w = make_workload("h3step", B=3, T=2, seq_lens=[900, 3000, 5000], bt_width=40, k=700, seed=33,
                      exp_range=(124, 127))
    H = 3
    rng = np.random.default_rng(34)
    kh = rng.integers(0, 256, size=(w.num_pages, H, 8704), dtype=np.uint8)
    vh = rng.integers(0, 256, size=(w.num_pages, H, 8704), dtype=np.uint8)
    kh[..., 8192:] = rng.integers(124, 128, size=(w.num_pages, H, 512))
    vh[..., 8192:] = rng.integers(124, 128, size=(w.num_pages, H, 512))
    w.k_pool, w.v_pool = kh, vh
    w.q = mxfp4.round_to_bf16_bits(rng.standard_normal((w.N, 16 * H, 128)))
    d = to_device(w)
    ws = spd.Workspace("cuda")
    out, sel = _step(spd, w, d, ws)
    assert spd.check_device_errors(ws) == 0
    sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
    for i in range(w.N):
        check_topk_row(sel_np[i], w, i, w.k)
        b = i // w.T
        pos = int(w.seq_lens[b]) - w.T + i % w.T
        for h in range(H):
            ref = decode.decode_one(w.q[i, 16 * h : 16 * h + 16], kh, vh, w.block_table[b], pos, w.scale, sel_np[i],
                                    head=h)
            vmax = float(np.abs(decode.sequence_rows(vh, w.block_table[b], pos + 1, h)).max())
            o = mxfp4.bf16_bits_to_f64(out_bits[i, 16 * h : 16 * h + 16])
            rel = np.linalg.norm(o - ref) / np.linalg.norm(ref)
            assert rel <= 5e-3 and np.max(np.abs(o - ref)) <= 1e-2 * vmax, (i, h, rel)


def _fixed_index_pool(w, codes):
    w.index_pool = mxfp4.pack(codes, np.full((w.num_pages, 128, 4), 127, dtype=np.uint8))


def test_step_one_token_all_equal_scores(spd):
    """One query token per request (chunks resolve the threshold among
    themselves) and every index score equal: the k lowest positions are
    selected; a request with fewer valid tokens than k takes them all."""
    w = make_workload("eqstep", B=3, T=1, seq_lens=[9000, 5000, 300], bt_width=71, k=1000, seed=41,
                      exp_range=(124, 127))
    _fixed_index_pool(w, np.full((w.num_pages, 128, 128), 2, dtype=np.uint8))
    d = to_device(w)
    ws = spd.Workspace("cuda")
    out, sel = _step(spd, w, d, ws)
    assert spd.check_device_errors(ws) == 0
    sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
    for i, L in enumerate(w.seq_lens):
        n = min(w.k, int(L))
        assert sorted(sel_np[i][:n].tolist()) == list(range(n)) and np.all(sel_np[i][n:] == -1), i
        _check_token(w, i, sel_np[i], out_bits)


def test_step_one_token_exact_ties_at_threshold(spd):
    """A few distinct score values, so every radix level ends in a bin of
    exact ties: the selection equals the oracle's, lowest positions first."""
    w = make_workload("tiestep", B=4, T=1, seq_lens=[3000, 7000, 12000, 640], bt_width=96, k=777, seed=42,
                      exp_range=(124, 127))
    rng = np.random.default_rng(43)
    codes = np.zeros((w.num_pages, 128, 128), dtype=np.uint8)
    codes[:, :, 0] = rng.integers(0, 8, size=(w.num_pages, 128))  # score = iq[0] * value
    _fixed_index_pool(w, codes)
    w.index_q[:, 0] = mxfp4.round_to_bf16_bits(np.array([1.0]))[0]
    d = to_device(w)
    ws = spd.Workspace("cuda")
    for rep in range(2):  # the second call reuses the workspace the first left clean
        out, sel = _step(spd, w, d, ws)
        assert spd.check_device_errors(ws) == 0
        sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
        for i, L in enumerate(w.seq_lens):
            pos = int(L) - 1
            ref = decode.topk(decode.index_scores(w.index_q[i], w.index_pool, w.block_table[i], pos), w.k)
            n = min(w.k, pos + 1)
            assert sorted(sel_np[i][:n].tolist()) == sorted(ref.tolist()), (rep, i)
            _check_token(w, i, sel_np[i], out_bits)


def test_step_one_token_small_tie_groups(spd):
    """512 distinct score values (v0 + v1/16 + v2/256 over e2m1 magnitudes),
    a few to a few dozen tokens each: the exchanged threshold bin ends in a
    small sub-bin of exact ties, split between selected and not (3 -> 1,
    18 -> 17, 19 -> 11 places), which goes to the lowest positions."""
    w = make_workload("ties512step", B=4, T=1, seq_lens=[3000, 7000, 12000, 640], bt_width=96, k=777, seed=45,
                      exp_range=(124, 127))
    rng = np.random.default_rng(46)
    codes = np.zeros((w.num_pages, 128, 128), dtype=np.uint8)
    codes[:, :, 0:3] = rng.integers(0, 8, size=(w.num_pages, 128, 3))
    _fixed_index_pool(w, codes)
    w.index_q[:, :] = 0
    w.index_q[:, 0:3] = mxfp4.round_to_bf16_bits(np.array([1.0, 1.0 / 16, 1.0 / 256]))
    d = to_device(w)
    ws = spd.Workspace("cuda")
    for rep in range(2):
        out, sel = _step(spd, w, d, ws)
        assert spd.check_device_errors(ws) == 0
        sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
        for i, L in enumerate(w.seq_lens):
            pos = int(L) - 1
            ref = decode.topk(decode.index_scores(w.index_q[i], w.index_pool, w.block_table[i], pos), w.k)
            n = min(w.k, pos + 1)
            assert sorted(sel_np[i][:n].tolist()) == sorted(ref.tolist()), (rep, i)
            _check_token(w, i, sel_np[i], out_bits)


def test_step_one_token_concentrated_threshold_bin(spd):
    """The tokens of the threshold bin sit in the first chunks only (more of
    them in one chunk than the exchange requests at once) and tie exactly:
    the k lowest positions of the tied tokens are selected.  A second request
    with fewer tokens than k takes all of them in the same launch."""
    w = make_workload("concstep", B=2, T=1, seq_lens=[4096, 250], bt_width=32, k=300, seed=47,
                      exp_range=(124, 127))
    codes = np.zeros((w.num_pages, 128, 128), dtype=np.uint8)
    rng = np.random.default_rng(48)
    codes[:, :, 0] = rng.integers(1, 4, size=(w.num_pages, 128))  # scores 0.5 .. 1.5 times iq[0]
    bt0 = w.block_table[0]
    for p in range(4):  # the first 512 positions of request 0 all score 6 * iq[0]
        codes[bt0[p], :, 0] = 7
    _fixed_index_pool(w, codes)
    w.index_q[:, 0] = mxfp4.round_to_bf16_bits(np.array([1.0]))[0]
    d = to_device(w)
    ws = spd.Workspace("cuda")
    out, sel = _step(spd, w, d, ws)
    assert spd.check_device_errors(ws) == 0
    sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
    assert sorted(sel_np[0].tolist()) == list(range(300))
    assert sorted(sel_np[1][:250].tolist()) == list(range(250)) and np.all(sel_np[1][250:] == -1)
    for i in range(2):
        _check_token(w, i, sel_np[i], out_bits)


def test_step_one_token_three_kv_heads(spd):
    """Three KV heads with one query token per request: every chunk attends
    over its selected tokens for each head."""
    w = make_workload("h3t1", B=3, T=1, seq_lens=[900, 3000, 5000], bt_width=40, k=700, seed=44,
                      exp_range=(124, 127))
    H = 3
    rng = np.random.default_rng(45)
    kh = rng.integers(0, 256, size=(w.num_pages, H, 8704), dtype=np.uint8)
    vh = rng.integers(0, 256, size=(w.num_pages, H, 8704), dtype=np.uint8)
    kh[..., 8192:] = rng.integers(124, 128, size=(w.num_pages, H, 512))
    vh[..., 8192:] = rng.integers(124, 128, size=(w.num_pages, H, 512))
    w.k_pool, w.v_pool = kh, vh
    w.q = mxfp4.round_to_bf16_bits(rng.standard_normal((w.N, 16 * H, 128)))
    d = to_device(w)
    out, sel = _step(spd, w, d, spd.Workspace("cuda"))
    sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
    for i in range(w.N):
        check_topk_row(sel_np[i], w, i, w.k)
        pos = int(w.seq_lens[i]) - 1
        for h in range(H):
            ref = decode.decode_one(w.q[i, 16 * h : 16 * h + 16], kh, vh, w.block_table[i], pos, w.scale, sel_np[i],
                                    head=h)
            vmax = float(np.abs(decode.sequence_rows(vh, w.block_table[i], pos + 1, h)).max())
            o = mxfp4.bf16_bits_to_f64(out_bits[i, 16 * h : 16 * h + 16])
            rel = np.linalg.norm(o - ref) / np.linalg.norm(ref)
            assert rel <= 5e-3 and np.max(np.abs(o - ref)) <= 1e-2 * vmax, (i, h, rel)


def test_step_one_token_mid_batch(spd):
    """40 requests of ragged length (12 chunks each, 480 resident chunk
    items): sampled tokens against the oracle, every selection valid."""
    w = make_workload("mid40", B=40, T=1, seq_lens=(6000, 16384), bt_width=128, k=1500, seed=46,
                      exp_range=(124, 127))
    d = to_device(w)
    ws = spd.Workspace("cuda")
    out, sel = _step(spd, w, d, ws)
    assert spd.check_device_errors(ws) == 0
    sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
    for i in range(0, w.N, 5):
        _check_token(w, i, sel_np[i], out_bits)
    for i, L in enumerate(w.seq_lens):
        row = sel_np[i]
        assert np.unique(row).size == w.k and np.all((row >= 0) & (row < L))


def test_one_workspace_across_formats_windows_and_inserts(spd):
    """One buffer for MXFP4 and fp8 steps, window scans, dense attention and
    inserts, in a mixed order: each result equals the same call on a fresh
    workspace."""
    ws = spd.Workspace("cuda", 64 << 20)
    w4 = make_workload("mix4", B=3, T=2, seq_lens=[700, 3000, 5000], bt_width=40, k=300, seed=81,
                       exp_range=(124, 127))
    w8 = make_workload("mix8", B=2, T=1, seq_lens=[9000, 130], bt_width=71, k=500, seed=82, cache="fp8")
    d4, d8 = to_device(w4), to_device(w8)

    def step4(ws_):
        return spd.mono_sparse_decode_mxfp4(d4["index_q"], d4["index_pool"], d4["q"], d4["k_pool"], d4["v_pool"],
                                            d4["block_table"], d4["seq_lens"], w4.k, w4.scale, T=w4.T, workspace=ws_)

    def step8(ws_):
        return spd.mono_sparse_decode_fp8(d8["index_q"], d8["index_pool"], d8["q"], d8["k_pool"], d8["v_pool"],
                                          d8["block_table"], d8["seq_lens"], w8.k, w8.scale, w8.k_scale, w8.v_scale,
                                          workspace=ws_)

    def window(ws_):
        return spd.mono_index_score_topk(d4["index_q"], d4["index_pool"], d4["block_table"], d4["seq_lens"], w4.k,
                                         T=w4.T, page_window=(10, 30), workspace=ws_)

    def dense(ws_):
        return spd.mono_pa_decode_mxfp4(d4["q"], d4["k_pool"], d4["v_pool"], d4["block_table"], d4["seq_lens"], None,
                                        w4.scale, T=w4.T, workspace=ws_)

    def norm(r):
        if isinstance(r, tuple):
            out, sel = r
            return bf16_bits(out), np.sort(sel.cpu().numpy(), axis=1)
        return (np.sort(r.cpu().numpy(), axis=1),) if r.dtype == torch.int32 else (bf16_bits(r),)

    calls = [step8, window, step4, dense, step8, step4, window]
    want = {f.__name__: norm(f(spd.Workspace("cuda"))) for f in set(calls)}
    torch.cuda.synchronize()
    for n, f in enumerate(calls):
        got = norm(f(ws))
        torch.cuda.synchronize()
        for a, b in zip(got, want[f.__name__]):
            if a.dtype == np.uint16:  # outputs: equal up to fp32 summation order
                fa, fb = mxfp4.bf16_bits_to_f64(a), mxfp4.bf16_bits_to_f64(b)
                assert np.max(np.abs(fa - fb)) <= 1e-2 * np.max(np.abs(fb)), (n, f.__name__)
            else:
                np.testing.assert_array_equal(a, b, err_msg=f"call {n} ({f.__name__})")
        # an insert into a copy of the pools reports its errors through the same workspace
        if n == 3:
            slots = torch.tensor([5, 3 * 10**9], dtype=torch.int64, device="cuda")
            rows = torch.zeros((2, 128), dtype=torch.bfloat16, device="cuda")
            spd.mono_insert_mxfp4(slots, index_rows=rows, index_pages=d4["index_pool"].clone(), workspace=ws)
            assert spd.check_device_errors(ws) == spd.DEVERR_SLOT
    assert spd.check_device_errors(ws) == 0


def test_shared_workspace_larger_record_then_chunk_local(spd):
    """One workspace: a four-token step (a large zero region), then a one-token
    chunk-local step of the same table width whose chunks exchange candidates
    (writing scratch inside the larger zero region), then the four-token step
    again.  The chunk-local call must lower the workspace's zero record so
    that the third call clears what it dirtied.  Each result equals the same
    call on a fresh workspace and the oracle."""
    ws = spd.Workspace("cuda", 64 << 20)
    w4 = make_workload("rec4", B=3, T=4, seq_lens=[700, 5000, 3100], bt_width=40, k=300, seed=61,
                       exp_range=(124, 127))
    w1 = make_workload("rec1", B=1, T=1, seq_lens=[5000], bt_width=40, k=300, seed=62, exp_range=(124, 127))
    d4, d1 = to_device(w4), to_device(w1)
    fresh = {}
    for name, w, d in (("rec4", w4, d4), ("rec1", w1, d1)):
        out, sel = _step(spd, w, d, spd.Workspace("cuda"))
        fresh[name] = (np.sort(sel.cpu().numpy(), axis=1), bf16_bits(out))
    for n, (name, w, d) in enumerate((("rec4", w4, d4), ("rec1", w1, d1), ("rec4", w4, d4), ("rec1", w1, d1))):
        out, sel = _step(spd, w, d, ws)
        assert spd.check_device_errors(ws) == 0, (n, name)
        sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
        np.testing.assert_array_equal(np.sort(sel_np, axis=1), fresh[name][0], err_msg=f"call {n} ({name})")
        for i in range(w.N):
            _check_token(w, i, sel_np[i], out_bits)
            assert_resplit_close(out_bits[i], fresh[name][1][i], resplit_bound(w, i, sel_np[i]), f"call {n} query {i}")


def test_chunk_local_step_equals_two_calls(spd):
    """One query token per request: the chunk-local launch (each chunk of a
    request attends over its own share of the selection, one split per
    chunk) against the index call followed by the attention call (splits of
    the selection list): the same sets, and outputs within the bound that the
    bf16 rounding of split-relative probabilities implies
    (helpers.resplit_bound)."""
    w = make_workload("cl2", B=6, T=1, seq_lens=[32768, 20000, 9000, 30001, 4097, 128 * 200], bt_width=256, k=2048,
                      seed=63, exp_range=(124, 127))
    d = to_device(w)
    out, sel = _step(spd, w, d, spd.Workspace("cuda"))
    sel2 = spd.mono_index_score_topk(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], w.k)
    out2 = spd.mono_pa_decode_mxfp4(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], sel2, w.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np.sort(sel2.cpu().numpy(), axis=1), np.sort(sel.cpu().numpy(), axis=1))
    sel_np, a, b = sel.cpu().numpy(), bf16_bits(out), bf16_bits(out2)
    for i in range(w.N):
        assert_resplit_close(a[i], b[i], resplit_bound(w, i, sel_np[i]), f"query {i}")
    sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
    for i in range(w.N):
        _check_token(w, i, sel_np[i], out_bits)
