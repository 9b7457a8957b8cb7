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


def check_topk_row(sel_row, w, i, k):
    """Acceptance check of one query token's selection against the oracle."""
    T = w.T
    b = i // T
    pos = int(w.seq_lens[b]) - T + i % T
    s = decode.index_scores(w.index_q[i], w.index_pool, w.block_table[b], pos)
    n = min(k, pos + 1)
    sel_row = np.asarray(sel_row)
    got = sel_row[:n]
    assert np.all(sel_row[n:] == -1), f"query {i}: padding is not -1"
    assert np.all((got >= 0) & (got <= pos)), f"query {i}: selection outside 0..{pos}"
    assert len(np.unique(got)) == n, f"query {i}: duplicate selections"
    ref = decode.topk(s, k)
    kth = np.sort(s)[::-1][n - 1]
    diff = np.setxor1d(got, ref)
    bad = diff[np.abs(s[diff] - kth) > TOPK_TIE_BAND * abs(kth)]
    assert bad.size == 0, (
        f"query {i}: {bad.size} tokens differ beyond the tie band; k-th score {kth!r}, "
        f"e.g. token {bad[0]} score {s[bad[0]]!r}"
    )
    return diff.size


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
