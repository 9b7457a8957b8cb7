"""GPU parity of the fp8 (e4m3) cache variant of the step against the oracle.

The same bars as the MXFP4 path: the page conversion bit-exact for all 256
codes; selections equal to the oracle's top-k up to exact-tie order (1e-6
relative band of the k-th score); attention within relative L2 5e-3 and
max |err| 1e-2 max|V| of the oracle's float64 decode with the K and V
tensor scales applied.
"""

import numpy as np
import pytest
import torch

from helpers import bf16_bits, check_topk_row, to_device
from oracle import decode, fp8, mxfp4
from workloads import make_workload, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_amd as spd

    spd.load_library()
    assert torch.cuda.is_available()
    return spd


def _step(spd, w, d, ws=None):
    out, sel = spd.mono_sparse_decode_fp8(d["index_q"], d["index_pool"], d["q"], d["k_pool"], d["v_pool"],
                                          d["block_table"], d["seq_lens"], w.k, w.scale, w.k_scale, w.v_scale, T=w.T,
                                          workspace=ws)
    torch.cuda.synchronize()
    return out, sel


def _check_attention(w, i, out_bits, sel_row=None):
    b = i // w.T
    pos = int(w.seq_lens[b]) - w.T + i % w.T
    ref = decode.decode_one(w.q[i], w.k_pool, w.v_pool, w.block_table[b], pos, w.scale, sel_row,
                            k_scale=w.k_scale, v_scale=w.v_scale)
    vmax = w.v_scale * float(np.abs(decode.sequence_rows(w.v_pool, w.block_table[b], pos + 1, 0)).max())
    o = mxfp4.bf16_bits_to_f64(out_bits[i])
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(o - ref) / nref if nref > 0 else np.linalg.norm(o)
    assert rel <= 5e-3 and np.max(np.abs(o - ref)) <= 1e-2 * vmax, (i, rel)


def test_fp8_dequant_bit_exact_all_codes(spd):
    rng = np.random.default_rng(40)
    codes = np.concatenate([rng.permutation(256) for _ in range(2 * fp8.PAGE_BYTES // 256)]).astype(np.uint8)
    pages = codes.reshape(2, fp8.PAGE_BYTES)
    got = bf16_bits(spd.fp8_pages_dequant_bf16(torch.from_numpy(pages).cuda()))
    want = fp8.dequant(pages)
    nan = np.isnan(want)
    got_f = mxfp4.bf16_bits_to_f64(got)
    np.testing.assert_array_equal(np.isnan(got_f), nan)
    np.testing.assert_array_equal(got[~nan], mxfp4.round_to_bf16_bits(want)[~nan])
    # the conversion is exact: the bf16 value is the e4m3 value
    np.testing.assert_array_equal(got_f[~nan], want[~nan])


SMALL = [
    # name, B, T, seq_lens, bt_width, k
    ("one_page", 1, 1, [100], 1, 10),
    ("k_ge_valid", 2, 1, [50, 129], 2, 200),
    ("k_one", 3, 1, [1, 128, 700], 6, 1),
    ("ragged_multi_token", 4, 4, [4, 300, 1000, 2049], 17, 37),
    ("several_chunks", 2, 1, [5000, 4097], 40, 700),
    ("t3_group", 2, 3, [640, 3001], 24, 250),
    ("wide_table_slices", 2, 1, [3000, 9000], 520, 700),
    ("wide_table_slices_t2", 2, 2, [5000, 9100], 520, 300),
]


@pytest.mark.parametrize("name,B,T,lens,W,k", SMALL, ids=[c[0] for c in SMALL])
def test_fp8_step_small(spd, name, B, T, lens, W, k):
    print(f"[fp8] step {name}", flush=True)
    w = make_workload(name, B=B, T=T, seq_lens=lens, bt_width=W, k=k, seed=sum(map(ord, name)) + 17, cache="fp8")
    d = to_device(w)
    ws = spd.Workspace("cuda")
    out, sel = _step(spd, w, d, ws)
    assert spd.check_device_errors(ws) == 0
    sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
    for i in range(w.N):
        check_topk_row(sel_np[i], w, i, w.k)
        _check_attention(w, i, out_bits, sel_np[i])
    # the index call selects the same sets
    sel2 = spd.mono_index_score_topk_fp8(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], w.k, T=w.T)
    np.testing.assert_array_equal(np.sort(sel2.cpu().numpy(), axis=1), np.sort(sel_np, axis=1))


def test_fp8_step_equals_two_calls(spd):
    w = make_workload("two_fp8", B=3, T=2, seq_lens=[3000, 5000, 4100], bt_width=40, k=512, seed=48, cache="fp8")
    d = to_device(w)
    out, sel = _step(spd, w, d)
    sel2 = spd.mono_index_score_topk_fp8(d["index_q"], d["index_pool"], d["block_table"], d["seq_lens"], w.k, T=w.T)
    out2 = spd.mono_pa_decode_fp8(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], sel2, w.scale,
                                  w.k_scale, w.v_scale, T=w.T)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np.sort(sel2.cpu().numpy(), axis=1), np.sort(sel.cpu().numpy(), axis=1))
    a = mxfp4.bf16_bits_to_f64(bf16_bits(out))
    b = mxfp4.bf16_bits_to_f64(bf16_bits(out2))
    assert np.max(np.abs(a - b)) <= 1e-2 * np.max(np.abs(b))


@pytest.mark.parametrize("T,lens", [(1, [1, 700, 4000]), (4, [4, 130, 3000])], ids=["t1", "t4"])
def test_fp8_dense_attention(spd, T, lens):
    w = make_workload(f"dense_fp8_{T}", B=3, T=T, seq_lens=lens, bt_width=32, k=0, seed=50 + T, cache="fp8",
                      k_scale=0.75, v_scale=2.0)
    d = to_device(w)
    ws = spd.Workspace("cuda")
    out = spd.mono_pa_decode_fp8(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], None, w.scale,
                                 w.k_scale, w.v_scale, T=w.T, workspace=ws)
    torch.cuda.synchronize()
    assert spd.check_device_errors(ws) == 0
    out_bits = bf16_bits(out)
    for i in range(w.N):
        _check_attention(w, i, out_bits)


def test_fp8_bad_tensor_scales_are_refused(spd):
    w = make_workload("bad_scale", B=1, T=1, seq_lens=[100], bt_width=1, k=8, seed=52, cache="fp8")
    d = to_device(w)
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("nan"), 1.0), (1.0, float("inf"))):
        with pytest.raises(spd.MonoError):
            spd.mono_sparse_decode_fp8(d["index_q"], d["index_pool"], d["q"], d["k_pool"], d["v_pool"],
                                       d["block_table"], d["seq_lens"], w.k, w.scale, ks, vs)
    # MXFP4-sized pages are refused by the fp8 calls
    with pytest.raises(ValueError):
        spd.mono_index_score_topk_fp8(d["index_q"], torch.zeros((2, 8704), dtype=torch.uint8, device="cuda"),
                                      d["block_table"], d["seq_lens"], w.k)


@pytest.mark.parametrize("number,samples", [(3, [0, 31, 63]), (4, [0, 3, 101, 511])])
def test_fp8_step_full_size_sampled(spd, number, samples):
    """The benchmark's shapes with fp8 pools."""
    print(f"[fp8] full size workload {number}", flush=True)
    w = workload(number, cache="fp8")
    d = to_device(w)
    ws = spd.Workspace("cuda")
    out, sel = _step(spd, w, d, ws)
    assert spd.check_device_errors(ws) == 0
    sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
    for i in samples:
        check_topk_row(sel_np[i], w, i, w.k)
        _check_attention(w, i, out_bits, sel_np[i])
    pos = decode.query_positions(w.seq_lens, w.T)
    for i in range(w.N):
        n = min(w.k, pos[i] + 1)
        row = sel_np[i]
        assert np.all(row[n:] == -1) and np.all((row[:n] >= 0) & (row[:n] <= pos[i]))
        assert np.unique(row[:n]).size == n
    assert torch.isfinite(out.float()).all()


def test_fp8_step_two_kv_heads(spd):
    w = make_workload("h2fp8", B=2, T=1, seq_lens=[2000, 4100], bt_width=40, k=600, seed=55, cache="fp8")
    H = 2
    rng = np.random.default_rng(56)
    def pool():
        bits = rng.integers(0, 256, size=(w.num_pages, H, fp8.PAGE_BYTES), dtype=np.uint8)
        exp = rng.integers(4, 11, size=bits.shape, dtype=np.uint8)
        return (bits & 0x87) | (exp << 3)
    w.k_pool, w.v_pool = pool(), pool()
    w.q = mxfp4.round_to_bf16_bits(rng.standard_normal((w.N, 16 * H, 128)))
    d = to_device(w)
    out, sel = _step(spd, w, d)
    sel_np, out_bits = sel.cpu().numpy(), bf16_bits(out)
    for i in range(w.N):
        check_topk_row(sel_np[i], w, i, w.k)
        pos = int(w.seq_lens[i]) - 1
        for h in range(H):
            ref = decode.decode_one(w.q[i, 16 * h : 16 * h + 16], w.k_pool, w.v_pool, w.block_table[i], pos, w.scale,
                                    sel_np[i], head=h, k_scale=w.k_scale, v_scale=w.v_scale)
            o = mxfp4.bf16_bits_to_f64(out_bits[i, 16 * h : 16 * h + 16])
            assert np.linalg.norm(o - ref) <= 5e-3 * np.linalg.norm(ref), (i, h)
