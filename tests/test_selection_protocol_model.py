"""A CPU model of the hand-off between filter slices and the resolving slice.

The item-queue selection of one query token runs as many workgroups (one
per slice of its score row) that share three counters and two global
lists; none of them waits for another.  Each slice
  1. reads the token's complete histogram and finds the bin B1 of the k-th
     largest key and the count `above` of keys in higher bins;
  2. takes a block of output slots (out_cnt) for its keys above B1 and a
     block of candidate slots (cand_cnt) for its keys in B1, one atomic each;
  3. stores its positions and (key, position) candidates into those blocks;
  4. waits until its stores are complete;
  5. arrives at the token's slice counter.  The last to arrive resets the
     three counters and resolves: it reads the count(B1) candidates, keeps
     the k - above largest by (key descending, position ascending) and
     writes them to slots above..k-1.

The model runs these steps for every slice of a row under a random
interleaving, with each store becoming visible at a random later point
(at the latest at step 4 of the slice that issued it), then checks that the
output is the exact top-k with ties to the lowest positions, that every slot
is written once, and that the counters are zero again, so a second launch on
the same memory also selects exactly.  The same model with step 4 removed
selects wrong tokens in some schedules, which shows that the interleavings
reach the orderings the wait rules out.
"""
import numpy as np
import pytest

HIST_SHIFT = 21  # the histogram bin is the key's top 11 bits


def score_key(s):
    """Order-preserving uint32 key of float32 scores (NaN maps to 0)."""
    u = np.asarray(s, dtype=np.float32).view(np.uint32).astype(np.uint64)
    k = np.where(u & 0x80000000, ~u & 0xFFFFFFFF, u | 0x80000000)
    return np.where(np.isnan(s), 0, k).astype(np.uint64)


class Memory:
    """Global memory whose stores become visible some time after they issue."""

    def __init__(self, rng):
        self.rng = rng
        self.words = {}
        self.pending = []  # (issuer, address, value)

    def store(self, who, addr, value):
        self.pending.append((who, addr, value))

    def settle_some(self):
        keep = []
        for p in self.pending:
            if self.rng.random() < 0.3:
                self.words[p[1]] = p[2]
            else:
                keep.append(p)
        self.pending = keep

    def complete(self, who):
        keep = []
        for p in self.pending:
            if p[0] == who:
                self.words[p[1]] = p[2]
            else:
                keep.append(p)
        self.pending = keep

    def load(self, addr):
        return self.words.get(addr)

    def atomic_add(self, addr, v):
        old = self.words.get(addr, 0)
        self.words[addr] = old + v
        return old


def kth_bin(hist, k):
    """Bin of the k-th largest key and the count of keys in higher bins."""
    above = 0
    for b in range(len(hist) - 1, -1, -1):
        if above + hist[b] >= k:
            return b, above, int(hist[b])
        above += int(hist[b])
    raise AssertionError("fewer than k keys")


def slice_program(mem, keys, s, slice_len, k, n_slices, out_log, wait_before_arrival):
    """One filter slice, as a generator that yields between its steps."""
    hist = np.bincount((keys >> HIST_SHIFT).astype(np.int64), minlength=2048)
    b1, above, in_b1 = kth_bin(hist, k)
    j0, j1 = s * slice_len, min((s + 1) * slice_len, len(keys))
    bins = keys[j0:j1] >> HIST_SHIFT
    hi = [j0 + x for x in np.nonzero(bins > b1)[0]]
    eq = [(int(keys[j0 + x]), j0 + x) for x in np.nonzero(bins == b1)[0]]
    yield
    base_hi = mem.atomic_add("out_cnt", len(hi)) if hi else 0
    base_c = mem.atomic_add("cand_cnt", len(eq)) if eq else 0
    yield
    for q, j in enumerate(hi):
        mem.store(s, ("out", base_hi + q), j)
        out_log.append(base_hi + q)
        if q % 7 == 0:
            yield
    for q, c in enumerate(eq):
        mem.store(s, ("cand", base_c + q), c)
        if q % 7 == 0:
            yield
    yield
    if wait_before_arrival:
        mem.complete(s)
    yield
    last = mem.atomic_add("filter_cnt", 1) == n_slices - 1
    if not last:
        return
    for name in ("filter_cnt", "out_cnt", "cand_cnt"):
        mem.words[name] = 0
    yield
    cands = [mem.load(("cand", x)) for x in range(in_b1)]
    if any(c is None for c in cands):
        cands = [c for c in cands if c is not None]  # a candidate that was not visible yet is lost
    cands.sort(key=lambda c: (-c[0], c[1]))
    for q, (_, j) in enumerate(cands[: k - above]):
        mem.store(s, ("out", above + q), j)
        out_log.append(above + q)
    mem.complete(s)


def run_launch(mem, keys, k, slice_len, rng, wait_before_arrival=True):
    n_slices = -(-len(keys) // slice_len)
    out_log = []
    progs = [slice_program(mem, keys, s, slice_len, k, n_slices, out_log, wait_before_arrival)
             for s in range(n_slices)]
    live = list(range(n_slices))
    while live:
        x = live[rng.integers(len(live))]
        try:
            next(progs[x])
        except StopIteration:
            live.remove(x)
        mem.settle_some()
    for p in list(mem.pending):  # the end of the launch makes every store visible
        mem.words[p[1]] = p[2]
    mem.pending = []
    out = [mem.load(("out", q)) for q in range(k)]
    return out, out_log


def exact_topk(keys, k):
    order = sorted(range(len(keys)), key=lambda j: (-int(keys[j]), j))
    return sorted(order[:k])


def make_keys(rng, n, mode):
    if mode == "normal":
        s = rng.standard_normal(n).astype(np.float32)
    elif mode == "ties":  # few distinct values: the threshold bin is one exact key
        s = rng.integers(0, 6, n).astype(np.float32)
    else:  # one exponent: everything in a handful of bins
        s = (1.0 + rng.random(n)).astype(np.float32)
    return score_key(s)


@pytest.mark.parametrize("mode", ["normal", "ties", "narrow"])
def test_protocol_selects_exactly_under_any_interleaving(mode):
    for seed in range(40):
        rng = np.random.default_rng(seed)
        n = int(rng.integers(300, 1500))
        k = int(rng.integers(1, n // 2))
        slice_len = int(rng.choice([64, 100, 256]))
        keys = make_keys(rng, n, mode)
        mem = Memory(rng)
        want = exact_topk(keys, k)
        for launch in range(2):  # the second launch runs on the counters the first left behind
            out, log = run_launch(mem, keys, k, slice_len, rng)
            assert sorted(log) == list(range(k)), (seed, launch, "every slot written exactly once")
            assert sorted(out) == want, (seed, launch)
            assert all(mem.words.get(c, 0) == 0 for c in ("filter_cnt", "out_cnt", "cand_cnt")), (seed, launch)


def test_protocol_without_the_wait_can_lose_candidates():
    wrong = 0
    for seed in range(60):
        rng = np.random.default_rng(1000 + seed)
        n = 1200
        keys = make_keys(rng, n, "narrow")
        k = 500
        mem = Memory(rng)
        out, _ = run_launch(mem, keys, k, 100, rng, wait_before_arrival=False)
        if sorted(x for x in out if x is not None) != exact_topk(keys, k):
            wrong += 1
    assert wrong > 0
