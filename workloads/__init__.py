"""Seeded synthetic inputs for sparse paged MXFP4 decode.

This module only draws random numbers and lays them out; it computes nothing
of the method.  It is the one piece shared by the oracle-side tests and the
GPU side: both take the same arrays from here and process them with their
own code.

Recipe (every workload, all draws from ``numpy.random.default_rng(seed)`` in
this order):

1. ``seq_lens``: fixed, or uniform integers in ``[lo, hi]``.
2. Pool layout: request b needs ``ceil(L_b / 128)`` pages; the pool holds
   exactly their sum plus ``extra_pages``.  A random permutation of the pool
   (or the identity) is cut into consecutive runs, one per request, which
   fill the request's block-table row; entries past its pages are -1.
3. K pages, V pages (``[P, 1, 8704]``) and, for sparse workloads, index-K
   pages (``[P, 8704]``).  Each page's first 8192 bytes (its packed e2m1
   data) are uniform bytes, i.e. two independent uniform 4-bit codes; its
   last 512 bytes (its e8m0 scales) are uniform integers in the exponent
   range.  Unused pool pages get the same distribution.
4. ``q`` (``[B*T, 16, 128]``) and, for sparse workloads, ``index_q``
   (``[B*T, 128]``): standard normal float32 rounded to bfloat16
   (round-to-nearest-even), stored as uint16 bit patterns.

With ``cache="fp8"`` step 3 draws fp8 (e4m3) pages instead (``[P, 1, 16384]``
and ``[P, 16384]``): every byte has a uniform sign bit, an exponent field
uniform in ``fp8_exp_range`` (at most 14, so no NaN code) and a uniform
3-bit mantissa; the workload also carries the K and V tensor scales
``k_scale`` / ``v_scale`` it was built with.
"""

from dataclasses import dataclass

import numpy as np

_DATA_REGION = 8192  # packed e2m1 bytes at the start of a page
_SCALE_REGION = 512  # e8m0 bytes at the end of a page
_TOKENS_PER_PAGE = 128
Q_HEADS = 16
HEAD_DIM = 128


@dataclass
class Workload:
    name: str
    B: int
    T: int
    k: int  # 0: dense (no index selection)
    scale: float
    seq_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, W]
    k_pool: np.ndarray  # uint8 [P, 1, 8704]
    v_pool: np.ndarray  # uint8 [P, 1, 8704]
    q: np.ndarray  # uint16 bf16 bits [B*T, 16, 128]
    index_pool: np.ndarray | None = None  # uint8 [P, 8704]
    index_q: np.ndarray | None = None  # uint16 bf16 bits [B*T, 128]
    cache: str = "mxfp4"  # or "fp8": pools of [.., 16384] e4m3 pages
    k_scale: float = 1.0  # fp8 K tensor scale
    v_scale: float = 1.0  # fp8 V tensor scale

    @property
    def N(self):
        return self.B * self.T

    @property
    def num_pages(self):
        return self.k_pool.shape[0]

    @property
    def sparse(self):
        return self.k > 0


def _bf16_bits(x):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _pages(rng, shape, exp_range):
    lo, hi = exp_range
    data = rng.integers(0, 256, size=(*shape, _DATA_REGION), dtype=np.uint8)
    scales = rng.integers(lo, hi + 1, size=(*shape, _SCALE_REGION), dtype=np.int64).astype(np.uint8)
    return np.concatenate([data, scales], axis=-1)


def _fp8_pages(rng, shape, exp_range):
    lo, hi = exp_range
    assert 0 <= lo <= hi <= 14
    n = (*shape, _TOKENS_PER_PAGE * HEAD_DIM)
    bits = rng.integers(0, 256, size=n, dtype=np.uint8)  # its sign bit and low 3 bits are used
    exp = rng.integers(lo, hi + 1, size=n, dtype=np.uint8)
    bits &= 0x87
    exp <<= 3
    bits |= exp
    return bits


def make_workload(
    name,
    *,
    B,
    T,
    seq_lens,
    bt_width,
    k,
    seed,
    exp_range=(122, 132),
    scale=1.0 / np.sqrt(128.0),
    identity_table=False,
    extra_pages=0,
    cache="mxfp4",
    fp8_exp_range=(4, 10),
    k_scale=0.5,
    v_scale=0.25,
):
    """Build one workload; ``seq_lens`` is an int, a list, or a ``(lo, hi)`` range tuple."""
    rng = np.random.default_rng(seed)
    if isinstance(seq_lens, tuple):
        lens = rng.integers(seq_lens[0], seq_lens[1] + 1, size=B, dtype=np.int64)
    else:
        lens = np.broadcast_to(np.asarray(seq_lens, dtype=np.int64), (B,)).copy()
    n_pages = (lens + _TOKENS_PER_PAGE - 1) // _TOKENS_PER_PAGE
    if int(n_pages.max(initial=0)) > bt_width:
        raise ValueError("block table too narrow for the sequence lengths")
    P = int(n_pages.sum()) + int(extra_pages)
    perm = np.arange(P) if identity_table else rng.permutation(P)
    bt = np.full((B, bt_width), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, : n_pages[b]] = perm[off : off + n_pages[b]]
        off += int(n_pages[b])
    if cache == "fp8":
        k_pool = _fp8_pages(rng, (P, 1), fp8_exp_range)
        v_pool = _fp8_pages(rng, (P, 1), fp8_exp_range)
        index_pool = _fp8_pages(rng, (P,), fp8_exp_range) if k > 0 else None
    else:
        assert cache == "mxfp4"
        k_pool = _pages(rng, (P, 1), exp_range)
        v_pool = _pages(rng, (P, 1), exp_range)
        index_pool = _pages(rng, (P,), exp_range) if k > 0 else None
    N = B * T
    q = _bf16_bits(rng.standard_normal((N, Q_HEADS, HEAD_DIM), dtype=np.float32))
    index_q = _bf16_bits(rng.standard_normal((N, HEAD_DIM), dtype=np.float32)) if k > 0 else None
    return Workload(
        name=name,
        B=B,
        T=T,
        k=k,
        scale=float(scale),
        seq_lens=lens.astype(np.int32),
        block_table=bt,
        k_pool=k_pool,
        v_pool=v_pool,
        q=q,
        index_pool=index_pool,
        index_q=index_q,
        cache=cache,
        k_scale=float(k_scale) if cache == "fp8" else 1.0,
        v_scale=float(v_scale) if cache == "fp8" else 1.0,
    )


# The five seeded workloads: (name, keyword arguments).  Seeds are 1000 + number.
WORKLOADS = {
    1: ("tiny_dense_b1_ctx256", dict(B=1, T=1, seq_lens=256, bt_width=2, k=0, identity_table=True)),
    # 32 x 64 pages taken from a permuted pool of 4096
    2: ("dense_b32_ctx8k", dict(B=32, T=1, seq_lens=8192, bt_width=64, k=0, extra_pages=2048)),
    3: ("sparse_b64_ctx32k_top2048", dict(B=64, T=1, seq_lens=32768, bt_width=256, k=2048)),
    4: (
        "multitoken_sparse_b128_t4_ctx16k-64k_top2048",
        dict(B=128, T=4, seq_lens=(16384, 65536), bt_width=512, k=2048),
    ),
    5: (
        "long_sparse_b8_ctx256k_top4096",
        dict(B=8, T=1, seq_lens=262144, bt_width=2048, k=4096, exp_range=(110, 140)),
    ),
}


def workload(number, seed=None, **overrides):
    """Workload ``number`` (1..5) with its default seed 1000 + number."""
    name, kw = WORKLOADS[number]
    kw = {**kw, **overrides}
    return make_workload(name, seed=1000 + number if seed is None else seed, **kw)


# --- new rows for the cache insert ------------------------------------------------
#
# Recipe (``numpy.random.default_rng(seed)``, in this order): for each of K
# ([n, heads, 128]), V ([n, heads, 128]) and the index key ([n, 128]),
# standard-normal float32 rows times 2**u with u uniform in [-6, 6] per row,
# rounded to bfloat16.  With ``specials``, every 32-element block then has,
# with probability 0.02 each, all its elements set to +0.0, all to -0.0, or
# its elements scaled by 2**-130 (bfloat16 subnormals), and each element with
# probability 0.002 is set to +-inf or NaN, and 0.002 to -0.0.
def _special_blocks(rng, x):
    blocks = x.reshape(-1, 32)
    r = rng.random(blocks.shape[0])
    blocks[r < 0.02] = 0.0
    blocks[(r >= 0.02) & (r < 0.04)] = -0.0
    tiny = (r >= 0.04) & (r < 0.06)
    blocks[tiny] *= np.float32(2.0**-130)
    e = rng.random(blocks.shape)
    blocks[e < 0.001] = np.inf
    blocks[(e >= 0.001) & (e < 0.0015)] = -np.inf
    blocks[(e >= 0.0015) & (e < 0.002)] = np.nan
    blocks[(e >= 0.002) & (e < 0.004)] = -0.0
    return blocks.reshape(x.shape)


def new_rows(seed, n, heads, *, specials=False):
    """bf16 bit patterns of new K, V ([n, heads, 128]) and index-key ([n, 128]) rows."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in (("k", (n, heads, HEAD_DIM)), ("v", (n, heads, HEAD_DIM)), ("index", (n, HEAD_DIM))):
        x = rng.standard_normal(shape, dtype=np.float32)
        x *= np.exp2(rng.uniform(-6, 6, size=shape[:-1] + (1,))).astype(np.float32)
        if specials:
            x = _special_blocks(rng, x)
        out[name] = _bf16_bits(x)
    return out


def decode_slots(w):
    """int64 slots of the T tokens being decoded of each request (flat b*T + t).

    Token j of request b is row j % 128 of page block_table[b, j // 128], so
    its slot (page * 128 + row) is block_table[b, j // 128] * 128 + j % 128.
    """
    slots = np.empty(w.B * w.T, dtype=np.int64)
    for b in range(w.B):
        for t in range(w.T):
            j = int(w.seq_lens[b]) - w.T + t
            slots[b * w.T + t] = int(w.block_table[b, j // _TOKENS_PER_PAGE]) * _TOKENS_PER_PAGE + j % _TOKENS_PER_PAGE
    return slots
