"""Shared test helpers: moving workloads to the GPU and the acceptance checks.

The acceptance bars:
* pages, codes, scales, dequantised values: bit-exact (NaN positions must
  match; -0.0 must be kept);
* top-k sets: same size min(k, valid), valid distinct entries, -1 padding,
  and every token in the symmetric difference with the oracle's set within
  1e-6 (relative) of the oracle's k-th score;
* attention (bf16 out): relative L2 <= 5e-3 over the whole output and
  max |err| <= 1e-2 * max|V| over the tokens any query sees.
"""

import numpy as np
import torch

from oracle import decode, mxfp4

TOPK_TIE_BAND = 1e-6
ATTN_REL_L2 = 5e-3
ATTN_MAX_ABS_FRAC = 1e-2
BF16_U = 2.0**-8  # unit roundoff of bfloat16 (8 significant bits, round to nearest)


def bf16_tensor(bits, device):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def to_device(w, device="cuda"):
    d = dict(
        k_pool=torch.from_numpy(w.k_pool).to(device),
        v_pool=torch.from_numpy(w.v_pool).to(device),
        q=bf16_tensor(w.q, device),
        block_table=torch.from_numpy(w.block_table).to(device),
        seq_lens=torch.from_numpy(w.seq_lens).to(device),
    )
    if w.index_pool is not None:
        d["index_pool"] = torch.from_numpy(w.index_pool).to(device)
        d["index_q"] = bf16_tensor(w.index_q, device)
    return d


def check_topk_scores(sel_row, s, pos, k, what=""):
    """Acceptance check of one query token's selection against the oracle,
    given the oracle's exact scores ``s`` of tokens 0..pos."""
    n = min(k, pos + 1)
    sel_row = np.asarray(sel_row)
    got = sel_row[:n]
    assert np.all(sel_row[n:] == -1), f"{what}: padding is not -1"
    assert np.all((got >= 0) & (got <= pos)), f"{what}: selection outside 0..{pos}"
    assert len(np.unique(got)) == n, f"{what}: duplicate selections"
    ref = decode.topk(s, k)
    kth = np.sort(s)[::-1][n - 1]
    diff = np.setxor1d(got, ref)
    bad = diff[np.abs(s[diff] - kth) > TOPK_TIE_BAND * abs(kth)]
    assert bad.size == 0, (
        f"{what}: {bad.size} tokens differ beyond the tie band; k-th score {kth!r}, "
        f"e.g. token {bad[0]} score {s[bad[0]]!r}"
    )
    return diff.size


def check_topk_row(sel_row, w, i, k):
    """Acceptance check of one query token's selection against the oracle."""
    T = w.T
    b = i // T
    pos = int(w.seq_lens[b]) - T + i % T
    s = decode.index_scores(w.index_q[i], w.index_pool, w.block_table[b], pos)
    return check_topk_scores(sel_row, s, pos, k, f"query {i}")


class RequestRows:
    """The oracle's dequantised rows of one request, computed once: index key
    (if the workload has one), K and V of one KV head, tokens 0..L-1."""

    def __init__(self, w, b, head=0, k_pool=None, v_pool=None):
        L = int(w.seq_lens[b])
        bt = w.block_table[b]
        self.L = L
        self.index = decode.sequence_rows(w.index_pool, bt, L) if w.index_pool is not None else None
        self.k = decode.sequence_rows(w.k_pool if k_pool is None else k_pool, bt, L, head)
        self.v = decode.sequence_rows(w.v_pool if v_pool is None else v_pool, bt, L, head)


def full_size_check(w, forms, requests=None):
    """Every query token of the given requests (default: all) against the
    oracle, for each (selection, output bits, label) in ``forms``: the
    selection (None: dense) under the tie band, then the attention output
    over that selection, per token and over the whole checked output.  The
    oracle's rows of a request are computed once for all forms.  Returns per
    form (rel L2 over the checked output, max |err| / max|V|, tokens)."""
    pos = decode.query_positions(w.seq_lens, w.T)
    acc = [[0.0, 0.0, 0.0, 0.0, 0] for _ in forms]  # err^2, ref^2, max err, max|V|, tokens
    for b in range(w.B) if requests is None else requests:
        rows = RequestRows(w, b)
        for t in range(w.T):
            i = b * w.T + t
            p = int(pos[i])
            s = None
            vm = float(np.abs(rows.v[: p + 1]).max()) * w.v_scale
            for (sel_np, out_bits, what), a in zip(forms, acc):
                sel_row = None
                if sel_np is not None:
                    if s is None:
                        s = decode.scores_of_rows(w.index_q[i], rows.index[: p + 1])
                    check_topk_scores(sel_np[i], s, p, w.k, f"{what} query {i}")
                    sel_row = sel_np[i]
                ref = decode.decode_rows(w.q[i], rows.k, rows.v, p, w.scale, sel_row, w.k_scale, w.v_scale)
                o = mxfp4.bf16_bits_to_f64(out_bits[i])
                e = float(np.max(np.abs(o - ref)))
                nref = float(np.linalg.norm(ref))
                rel = float(np.linalg.norm(o - ref)) / nref if nref > 0 else float(np.linalg.norm(o))
                assert rel <= ATTN_REL_L2 and e <= ATTN_MAX_ABS_FRAC * vm, (
                    f"{what} query {i}: relative L2 {rel:.3e}, max |err| {e:.3e} = {e / vm:.3e} max|V|")
                a[0] += float(np.sum((o - ref) ** 2))
                a[1] += nref**2
                a[2] = max(a[2], e)
                a[3] = max(a[3], vm)
                a[4] += 1
    res = []
    for (_, _, what), (e2, r2, me, vmax, n) in zip(forms, acc):
        rel_all = (e2 / r2) ** 0.5 if r2 > 0 else e2**0.5
        assert rel_all <= ATTN_REL_L2 and me <= ATTN_MAX_ABS_FRAC * vmax, (what, rel_all, me, vmax)
        res.append((rel_all, me / max(vmax, 1e-300), n))
    return res


def attention_errors(out_gpu_bits, ref, v_max):
    o = mxfp4.bf16_bits_to_f64(out_gpu_bits)
    rel = np.linalg.norm(o - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.max(np.abs(o - ref)) if o.size else 0.0
    return rel, mx, mx / max(v_max, 1e-300)


def max_abs_v(w, n_tokens_per_seq):
    """max |dequantised V| over the tokens 0..n-1 of each request."""
    m = 0.0
    for b in range(w.B):
        rows = decode.sequence_rows(w.v_pool, w.block_table[b], int(n_tokens_per_seq[b]), 0)
        if rows.size:
            m = max(m, float(np.nanmax(np.abs(rows))))
    return m


def assert_attention_close(out_gpu, ref, v_max, what=""):
    rel, mx, frac = attention_errors(bf16_bits(out_gpu), ref, v_max)
    assert rel <= ATTN_REL_L2, f"{what}: relative L2 {rel:.3e} > {ATTN_REL_L2}"
    assert frac <= ATTN_MAX_ABS_FRAC, f"{what}: max abs err {mx:.3e} = {frac:.3e} max|V|"
    return rel, frac


def resplit_bound(w, i, sel_row):
    """Per-element bound ``[16, 128]`` on the difference between two bf16
    attention outputs of query token i that split the same candidates into
    different partial sums.

    The kernels round each probability to bf16 relative to the running
    maximum of its split, a relative error of at most u = 2^-8 (bf16 has 8
    significant bits), and normalise with the same rounded values, so an
    output element moves from the exact one by at most
    u * sum_j p_j |v_j - o| (p, o: the oracle's weights and output); two
    such outputs differ by twice that.  Added: fp32 summation of the n
    candidates and the rescalings, (n + 16) * 2^-24 * sum_j p_j |v_j|.  The
    caller adds the final bf16 roundings, u times each output's magnitude."""
    b = i // w.T
    pos = int(w.seq_lens[b]) - w.T + i % w.T
    cand = decode.candidates(pos, sel_row)
    n = int(cand.max()) + 1 if cand.size else 0
    k = decode.sequence_rows(w.k_pool, w.block_table[b], n, 0)[cand] * w.k_scale
    v = decode.sequence_rows(w.v_pool, w.block_table[b], n, 0)[cand] * w.v_scale
    if cand.size == 0:
        return np.zeros((16, 128))
    p = decode.softmax_weights(w.q[i], k, w.scale)
    o = p @ v
    spread = np.einsum("hj,hjd->hd", p, np.abs(v[None, :, :] - o[:, None, :]))
    return 2.0 * BF16_U * spread + (cand.size + 16) * 2.0**-24 * (p @ np.abs(v))


def assert_resplit_close(a_bits, b_bits, bound, what=""):
    a = mxfp4.bf16_bits_to_f64(a_bits)
    b = mxfp4.bf16_bits_to_f64(b_bits)
    lim = bound + BF16_U * (np.abs(a) + np.abs(b))
    bad = np.abs(a - b) > lim
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} elements differ beyond the re-split bound "
        f"(worst |a-b|/bound {float(np.max(np.abs(a - b) / lim)):.3f})")
    return float(np.mean(a == b))
