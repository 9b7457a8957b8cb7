"""Decode-step benchmark of the sparse paged MXFP4 decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--cache mxfp4|fp8]

A step is one pass of the whole path over one batch: on sparse workloads one
mono_sparse_decode_mxfp4 call (index scores, top-k and attention over the
selected tokens, in one launch); dense workloads run mono_pa_decode_mxfp4
alone.  The default workload is batch 64, context 32768 (256 pages per
request), top-2048.  ``--cache fp8`` runs the same shapes over the older
build's fp8 (e4m3) pages with the *_fp8 calls.

Inputs are resident in HBM before timing starts.  The K, V and index-key
pools are replicated ``--copies`` times and the steps rotate through the
copies, so each step reads pages that are not in the 256 MB Infinity Cache.

Printed (one JSON line): achieved HBM GB/s over the KV+index bytes the method
must read (the index rows of every valid token once per request, the K and V
rows of every selected token once per request) and the step time, both from
the timed region (K steps back to back between two events); the spread of
single steps from a second pass with an event pair around each step; the
roofline entry of the step kernel, timed in a further pass of the same steps
with HIP events recorded around each launch on its stream; the two-call form of the step (index call, then attention call)
timed the same way, for reference; the MXFP4 cache insert (the decoded
tokens' K, V and index-key rows written through their slots, and a
32768-token prefill-sized insert) by kernel time; the indexer's
context-parallel emulation (4 index heads over 4 page-window shards, then the
merge) by kernel time; and the CPU oracle timed on a bounded sample of the
same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E peak, GB/s
ROW_BYTES = {"mxfp4": 68, "fp8": 128}  # per token row: 64 B e2m1 + 4 B e8m0; or 128 B of e4m3
METRIC = "decode-step µs + achieved HBM GB/s (% of peak), B=64 ctx=32k top-2048"
CSRC = os.path.join(ROOT, "sparse_paged_decode_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# Source files that define each kernel; their digest keys the stored counter data.
_STEP_SOURCES = ["step.hip", "topk_device.h", "attn_device.h", "device_common.h", "block_ops.h", "launch.h",
                 "page_format.h", "plan.h", "plan.cpp"]
KERNEL_SOURCES = {
    "sparse_decode_kernel": _STEP_SOURCES,
    "index_topk_kernel": _STEP_SOURCES,
    "pa_decode_kernel": _STEP_SOURCES,
    "sparse_decode_fp8_kernel": _STEP_SOURCES,
    "pa_decode_fp8_kernel": _STEP_SOURCES,
    "insert_kernel": ["pages.hip", "device_common.h", "launch.h"],
}


def kernel_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload_name):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload_name}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != kernel_digest(kernel):
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    p.add_argument("--cache", default="mxfp4", choices=["mxfp4", "fp8"],
                   help="cache page format (fp8: the older build's e4m3 pages, same shapes)")
    p.add_argument("--copies", type=int, default=4, help="pool replicas rotated over (1 = warm cache)")
    p.add_argument("--cpu-sample", type=int, default=64, help="query tokens timed on the CPU oracle (0 = skip)")
    p.add_argument("--skip-graph", action="store_true", help="do not time the HIP-graph replays")
    p.add_argument("--skip-insert", action="store_true", help="do not time the cache insert")
    p.add_argument("--skip-cp", action="store_true", help="do not time the indexer context-parallel emulation")
    p.add_argument("--skip-scan-variants", action="store_true",
                   help="do not time the index scan on the matrix cores against the same scan on the VALU")
    p.add_argument("--skip-clocks", action="store_true",
                   help="do not sample the clocks under load (about one second of extra steps)")
    p.add_argument("--skip-ceilings", action="store_true",
                   help="do not time the read-bandwidth references over the index pool")
    p.add_argument("--skip-two-call", action="store_true",
                   help="do not time the two-call form of the step (profiling runs count one kernel only)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 128 MiB device copy 10 times (counter calibration) and exit")
    p.add_argument("--timeline", type=int, default=0, metavar="N",
                   help="only print the phase timeline of N launches from the trace build of the library "
                        "(libmono_decode_trace.so) and exit")
    return p.parse_args()


def copy_calibration():
    """A plain copy of known size, to calibrate rocprofv3's FETCH_SIZE/WRITE_SIZE."""
    import torch

    n = 128 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 10}))


# Phase stamps of the trace build (include/mono_trace.h), by item kind, in
# program order.
_ATTN_PHASES = {10: "attention: entry", 11: "attention: q and table loaded", 12: "attention: pass done",
                13: "attention: partials stored", 14: "attention: partials complete", 15: "attention: arrived",
                16: "attention: merged (last split)"}
TIMELINE_PHASES = {
    "chunk-local chunk": {2: "scan and histogram flush done", 3: "histogram complete (barrier)",
                          4: "threshold bin found", 5: "threshold-bin pairs stored",
                          6: "pairs complete (barrier)", 7: "pairs in LDS", 8: "k-th key found",
                          9: "selection list built", **_ATTN_PHASES},
    "scan": {7: "scan done (filtering locally)", 6: "row histogram complete (filtering locally)",
             2: "scores (or the local slice) complete", 3: "arrived at the group (or slice) counter",
             4: "resolve: final splits published", 5: "resolve: done", 17: "row selected (inline)"},
    "filter slice": {2: "slice filtered", 3: "arrived at the row counter", 4: "resolve: final splits published",
                     5: "resolve: done"},
    "attention split": dict(_ATTN_PHASES),
    "attention split, gated": {10: "attention: entry", 11: "attention: q, table, ready word, entries", 12: "attention: pass done",
                               13: "attention: partials stored", 14: "attention: partials complete",
                               15: "attention: arrived", 16: "attention: merged (last split)"},
    "selection": {17: "row selected"},
    "clear": {},
}


def timeline(args):
    """Phase timeline of the step from the trace build: p10/p50/p90/max of
    every stamp (us from the launch's first kernel entry) and the p50 step
    from the previous stamp of the same item, per item kind."""
    import ctypes

    import torch

    import sparse_paged_decode_amd as spd
    from sparse_paged_decode_amd.build import TRACE_LIB_PATH
    from workloads import workload

    lib = spd.load_library(TRACE_LIB_PATH)
    lib.mono_trace_clear.restype = ctypes.c_int
    lib.mono_trace_read.restype = ctypes.c_int
    lib.mono_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t]
    dev = torch.device("cuda:0")
    w = workload(args.workload, cache=args.cache)
    copies = max(1, args.copies)
    run = StepRunner(spd, torch, dev, w, copies)
    for s in range(max(args.warmup, copies)):
        run.step(s % copies)
    torch.cuda.synchronize(dev)
    n_items, n_groups = 8192 * 32, 4096 * 32
    print(f"# phase timeline of {w.name} ({args.cache} caches, {copies} pool copies rotated), trace build "
          f"(libmono_decode_trace.so: thread 0 of each workgroup stamps the 100 MHz device clock)")
    print(f"# command (repo root): python3 -u bench.py {' '.join(sys.argv[1:])}")
    print("# us from the launch's first kernel entry; 'step' = p50 of the time since the previous stamp of the same item")
    for launch in range(args.timeline):
        if lib.mono_trace_clear() != 0:
            raise RuntimeError("mono_trace_clear failed")
        run.step(launch % copies)
        torch.cuda.synchronize(dev)
        items = np.zeros(n_items, dtype=np.uint64)
        groups = np.zeros(n_groups, dtype=np.uint64)
        if lib.mono_trace_read(items.ctypes.data, n_items, groups.ctypes.data, n_groups) != 0:
            raise RuntimeError("mono_trace_read failed")
        print_timeline(launch, items.reshape(8192, 32).astype(np.int64), groups.reshape(4096, 32).astype(np.int64))


def print_timeline(launch, it, gr):
    """Prints one launch's records (item records it[t, s], workgroup records
    gr[w, s], as mono_trace_read returns them)."""
    entry = gr[:, 0][gr[:, 0] > 0]
    leave = gr[:, 1][gr[:, 1] > 0]
    t0 = entry.min()
    us = lambda v: (v - t0) / 100.0
    print(f"\n== launch {launch}: {entry.size} workgroups enter over {us(entry.max()):.2f} us; "
          f"the last leaves the item loop at {us(leave.max()):.2f} us")
    used = it[:, 0] > 0
    kinds = (it[:, 31] >> 24) & 0xFF
    local = bool(((kinds == 1) & used & (it[:, 10] > 0)).any())  # chunk-local chunks run attention
    names = {1: "chunk-local chunk" if local else "scan", 2: "filter slice", 3: "attention split",
             5: "attention split, gated", 4: "selection", 0xFF: "clear"}
    for kind, label in names.items():
        rec = it[used & (kinds == kind)]
        if rec.shape[0] == 0:
            continue
        phases = {0: "start", **TIMELINE_PHASES[label], 1: "end"}
        print(f"  {label}: {rec.shape[0]} items")
        print(f"    {'phase':38s} {'n':>5s} {'p10':>7s} {'p50':>7s} {'p90':>7s} {'max':>7s} {'step':>7s}")
        # Stamps in program order: the start, the kind's phases as listed, the end.
        order = [0] + [k for k in phases if k > 1] + [1]
        last = np.zeros(rec.shape[0], dtype=np.int64)  # each item's latest stamp so far
        for k in order:
            v = rec[:, k]
            ok = v > 0
            if not ok.any():
                continue
            a = us(v[ok])
            both = ok & (last > 0)
            step = f"{np.median((v[both] - last[both]) / 100.0):7.2f}" if both.any() else ""
            print(f"    {phases[k]:38s} {ok.sum():5d} {np.percentile(a, 10):7.2f} {np.percentile(a, 50):7.2f} "
                  f"{np.percentile(a, 90):7.2f} {a.max():7.2f} {step:>7s}")
            last = np.where(ok, v, last)
        # First-round items by compute-unit slot: with two resident
        # workgroups per CU, tickets below half the grid are the first
        # workgroup dispatched to their CU.
        tickets = np.nonzero(used & (kinds == kind))[0]
        half = entry.size // 2
        first = (tickets < half) & (rec[:, 2] > 0)
        second = (tickets >= half) & (tickets < entry.size) & (rec[:, 2] > 0)
        # The XCD of a first-round item is its ticket mod 8 (workgroups are
        # dealt to the XCDs in turn).
        fr = tickets < entry.size
        if fr.sum() >= 8 and kind != 0xFF:
            ends = [rec[fr & (tickets % 8 == x), 1] for x in range(8)]
            ends = [us(e[e > 0]) for e in ends]
            print("    item end by XCD (first-round items), p50 / max: "
                  + ", ".join(f"{x}: {np.median(e):.1f} / {e.max():.1f}" for x, e in enumerate(ends) if e.size))
        if first.any() and second.any() and 2 in phases:
            d = (rec[:, 2] - rec[:, 0]) / 100.0
            print(f"    {phases[2]} after the start, p50: {np.median(d[first]):.2f} us for tickets below {half} "
                  f"(the first workgroup of each CU), {np.median(d[second]):.2f} us for tickets {half}..{entry.size - 1}")


def _read_text(path):
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return None


def _pci_dir(props):
    path = f"/sys/bus/pci/devices/{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}.0"
    return path if os.path.isdir(path) else None


def _dpm_levels(text):
    """(levels in MHz, index of the current level) of a pp_dpm_* file."""
    levels, cur = [], None
    for line in (text or "").splitlines():
        parts = line.replace(":", " ").split()
        if len(parts) >= 2 and parts[1].lower().endswith("mhz"):
            try:
                levels.append(int(parts[1][:-3]))
            except ValueError:
                continue
            if line.rstrip().endswith("*"):
                cur = len(levels) - 1
    return levels, cur


def device_info(torch, dev):
    """The GPU's identity: name, arch, compute units, memory, and from sysfs
    (when readable) its PCI device id, product name and clock levels."""
    props = torch.cuda.get_device_properties(dev)
    info = {"name": props.name, "arch": props.gcnArchName, "compute_units": props.multi_processor_count,
            "memory_GiB": round(props.total_memory / 2**30, 1)}
    d = _pci_dir(props)
    if d:
        info["pci"] = os.path.basename(d)
        for key, fname in (("pci_device_id", "device"), ("pci_revision", "revision"),
                           ("product_name", "product_name")):
            v = _read_text(os.path.join(d, fname))
            if v:
                info[key] = v
        for key, fname in (("sclk_levels_MHz", "pp_dpm_sclk"), ("mclk_levels_MHz", "pp_dpm_mclk")):
            levels, _ = _dpm_levels(_read_text(os.path.join(d, fname)))
            if levels:
                info[key] = levels
    return info, d


def clocks_under_load(pci_dir, run_steps, seconds=1.0):
    """Current sclk/mclk levels sampled from sysfs every 2 ms while steps run
    back to back for about `seconds` (a thread of this process reads the
    files; nothing is started).  None when sysfs does not expose them."""
    import threading

    if not pci_dir or not os.path.exists(os.path.join(pci_dir, "pp_dpm_sclk")):
        return None
    samples = {"sclk": [], "mclk": []}
    stop = threading.Event()

    def sample():
        while not stop.is_set():
            for key in samples:
                levels, cur = _dpm_levels(_read_text(os.path.join(pci_dir, f"pp_dpm_{key}")))
                if cur is not None:
                    samples[key].append(levels[cur])
            time.sleep(0.002)

    th = threading.Thread(target=sample)
    th.start()
    try:
        run_steps(seconds)
    finally:
        stop.set()
        th.join()
    out = {}
    for key, v in samples.items():
        if v:
            out[f"{key}_MHz_median"] = float(np.median(v))
            out[f"{key}_MHz_max"] = int(max(v))
            out[f"{key}_samples"] = len(v)
    return out or None


def algorithmic_bytes(w, sel):
    """(index bytes, K+V bytes) the step must read: one row (68 B MXFP4, 128 B
    fp8) per index row of every valid token once per request, 2 rows per
    selected (or, dense, valid) token once per request (union over the
    request's query tokens)."""
    row = ROW_BYTES[w.cache]
    idx_bytes = int(np.sum(w.seq_lens.astype(np.int64))) * row if w.sparse else 0
    kv_tokens = 0
    for b in range(w.B):
        if sel is None:
            kv_tokens += int(w.seq_lens[b])
        else:
            rows = sel[b * w.T : (b + 1) * w.T]
            kv_tokens += int(np.unique(rows[rows >= 0]).size)
    return idx_bytes, 2 * row * kv_tokens


def cpu_baseline(w, n_sample):
    """The oracle (numpy float64) on the first n_sample query tokens, scaled to GB/s."""
    from oracle import decode

    threads = len(os.sched_getaffinity(0))
    pos = decode.query_positions(w.seq_lens, w.T)
    row = ROW_BYTES[w.cache]
    n = min(n_sample, w.N)
    t0 = time.perf_counter()
    done_bytes = 0
    for i in range(n):
        b = i // w.T
        bt = w.block_table[b]
        sel = None
        if w.sparse:
            s = decode.index_scores(w.index_q[i], w.index_pool, bt, pos[i])
            sel = decode.topk(s, w.k)
            done_bytes += (pos[i] + 1) * row
        decode.decode_one(w.q[i], w.k_pool, w.v_pool, bt, pos[i], w.scale, sel, k_scale=w.k_scale, v_scale=w.v_scale)
        done_bytes += 2 * row * (len(sel) if sel is not None else pos[i] + 1)
    dt = time.perf_counter() - t0
    return {
        "value": round(done_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n} of {w.N} query tokens of {w.name} (scores + top-k + attention per query token), "
        f"{dt:.1f} s; numpy float64, BLAS threads <= {threads}",
    }


def insert_bytes(n, heads):
    """Algorithmic HBM bytes of inserting n tokens into K, V (heads each) and the index key.

    Per written row: 256 B of bf16 read, 64 B of e2m1 and 4 B of scales
    written; per token: its 8-B slot.
    """
    rows = n * (2 * heads + 1)
    return rows * (256 + 68) + 8 * n


def time_insert(spd, torch, dev, w, kp, vp, ip, reps):
    """Kernel time of the cache insert: the step's own decoded tokens and a 32768-token prefill."""
    from workloads import decode_slots, new_rows

    H = kp[0].shape[1]
    res = {}
    for name, n, slots in (("decode", w.N, decode_slots(w)), ("prefill_32768", 32768, np.arange(32768, dtype=np.int64))):
        r = new_rows(77, n, H)
        rows = {c: torch.from_numpy(r[c].view(np.int16)).view(torch.bfloat16).to(dev) for c in r}
        sl = torch.from_numpy(slots).to(dev)
        ws = spd.Workspace(dev)

        def ins(c):
            spd.mono_insert_mxfp4(sl, k_rows=rows["k"], v_rows=rows["v"], index_rows=rows["index"],
                                  k_pages=kp[c], v_pages=vp[c], index_pages=ip[c], workspace=ws)

        for s in range(5):
            ins(s % len(kp))
        torch.cuda.synchronize(dev)
        with spd.KernelTimer(capacity=reps + 4) as kt:
            for s in range(reps):
                ins(s % len(kp))
            torch.cuda.synchronize(dev)
        assert spd.check_device_errors(ws) == 0
        us = kt.mean_us["insert_kernel"]
        nbytes = insert_bytes(n, H)
        res[name] = {"tokens": n, "kernel_us_mean": round(us, 3), "algorithmic_bytes": nbytes,
                     "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    return res


def time_cp(spd, torch, dev, w, iq, ip, bt, sl, reps, heads=4):
    """Kernel times of the indexer context-parallel emulation: `heads` index heads over `heads` shards.

    One shard launch scores its page window of every request for all heads
    (the work one rank of the context-parallel indexer does); the merge keeps
    each head's top-k.  For reference, the one-head index call over whole
    sequences (the work without context parallelism, per head).
    """
    rng = np.random.default_rng(90)
    extra = torch.from_numpy(rng.standard_normal((heads - 1, w.N, 128), dtype=np.float32)).to(dev).to(torch.bfloat16)
    q_heads = torch.cat([iq[None], extra]).contiguous()
    ws = spd.Workspace(dev)
    for _ in range(3):
        spd.indexer_cp_topk(q_heads, ip, bt, sl, w.k, T=w.T, shards=heads, workspace=ws)
    torch.cuda.synchronize(dev)
    with spd.KernelTimer(capacity=(heads + 1) * reps + 8) as kt:
        for _ in range(reps):
            spd.indexer_cp_topk(q_heads, ip, bt, sl, w.k, T=w.T, shards=heads, workspace=ws)
        torch.cuda.synchronize(dev)
    W = bt.shape[1]
    lens = w.seq_lens.astype(np.int64)
    win_bytes = []
    for lo, hi in spd.cp_shard_windows(W, heads):
        toks = np.clip(lens, lo * 128, hi * 128) - lo * 128
        win_bytes.append(int(toks.sum()) * ROW_BYTES["mxfp4"])
    shard_us = kt.mean_us["index_topk_kernel"]
    merge_us = kt.mean_us["topk_merge_kernel"]
    return {
        "heads": heads,
        "shards": heads,
        "shard_kernel_us_mean": round(shard_us, 2),
        "merge_kernel_us_mean": round(merge_us, 2),
        "call_kernel_us": round(heads * shard_us + merge_us, 2),
        "shard_index_bytes": max(win_bytes),
        "shard_gbps": round(max(win_bytes) / shard_us / 1e3, 1),
        "note": "one launch per shard scores its page window for every head (up to four (head, token) rows per "
                "MFMA tile, so each window page is read once); the merge keeps each head's top-k",
    }


def time_scan_variants(spd, torch, dev, w, iq, ip, bt, sl, reps, chunk_pages=32):
    """The scan phase on the matrix cores and on the VALU (same reads, same
    LDS scores and histograms): kernel times and read rates."""
    hist = torch.zeros((w.B, 2048), dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    q1 = iq.view(w.B, w.T, 128)[:, -1].contiguous()  # each request's last query token
    out = {}
    for variant, name in ((0, "mfma"), (1, "valu")):
        for _ in range(3):
            spd.bench_scan(q1, ip, bt, sl, chunk_pages, variant, hist=hist, err=err)
        torch.cuda.synchronize(dev)
        with spd.KernelTimer(capacity=reps + 8) as kt:
            for _ in range(reps):
                spd.bench_scan(q1, ip, bt, sl, chunk_pages, variant, hist=hist, err=err)
            torch.cuda.synchronize(dev)
        us = kt.mean_us[f"scan_{name}_kernel"]
        out[f"{name}_kernel_us"] = round(us, 2)
    toks = int(np.clip(w.seq_lens.astype(np.int64), 0, None).sum())
    nbytes = toks * ROW_BYTES["mxfp4"]
    out["index_bytes"] = nbytes
    out["mfma_gbps"] = round(nbytes / out["mfma_kernel_us"] / 1e3, 1)
    out["valu_gbps"] = round(nbytes / out["valu_kernel_us"] / 1e3, 1)
    out["chunk_pages"] = chunk_pages
    return out


class StepRunner:
    """One workload's inputs in HBM and its step.

    The K, V and index-key pools are replicated ``copies`` times; ``step(c)``
    runs one step over copy c: on sparse workloads one
    mono_sparse_decode_{mxfp4,fp8} call, on dense ones mono_pa_decode_* alone.
    ``two_calls(c)`` is the same step as the index call followed by the
    attention call.  Outputs go to ``out`` / ``sel`` unless others are given.
    """

    def __init__(self, spd, torch, dev, w, copies):
        self.spd, self.w = spd, w
        self.f8 = w.cache == "fp8"

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        self.q = bf16(w.q)
        self.bt = torch.from_numpy(w.block_table).to(dev)
        self.sl = torch.from_numpy(w.seq_lens).to(dev)
        self.iq = bf16(w.index_q) if w.sparse else None
        self.kp = [torch.from_numpy(w.k_pool).to(dev)]
        self.vp = [torch.from_numpy(w.v_pool).to(dev)]
        self.ip = [torch.from_numpy(w.index_pool).to(dev)] if w.sparse else [None]
        for _ in range(copies - 1):
            self.kp.append(self.kp[0].clone())
            self.vp.append(self.vp[0].clone())
            self.ip.append(self.ip[0].clone() if w.sparse else None)
        self.copies = copies
        self.sel = torch.empty((w.N, w.k), dtype=torch.int32, device=dev) if w.sparse else None
        self.out = torch.empty_like(self.q)
        self.ws = spd.Workspace(dev)
        self.ws_topk = spd.Workspace(dev)
        self.ws_pa = spd.Workspace(dev)

    def step(self, c, out=None, sel=None):
        spd, w = self.spd, self.w
        out = self.out if out is None else out
        sel = self.sel if sel is None else sel
        iq, q, bt, sl, kp, vp, ip = self.iq, self.q, self.bt, self.sl, self.kp[c], self.vp[c], self.ip[c]
        if w.sparse and self.f8:
            spd.mono_sparse_decode_fp8(iq, ip, q, kp, vp, bt, sl, w.k, w.scale, w.k_scale, w.v_scale, T=w.T,
                                       out=out, selected_idx=sel, workspace=self.ws)
        elif w.sparse:
            spd.mono_sparse_decode_mxfp4(iq, ip, q, kp, vp, bt, sl, w.k, w.scale, T=w.T, out=out, selected_idx=sel,
                                         workspace=self.ws)
        elif self.f8:
            spd.mono_pa_decode_fp8(q, kp, vp, bt, sl, None, w.scale, w.k_scale, w.v_scale, T=w.T, out=out,
                                   workspace=self.ws_pa)
        else:
            spd.mono_pa_decode_mxfp4(q, kp, vp, bt, sl, None, w.scale, T=w.T, out=out, workspace=self.ws_pa)

    def two_calls(self, c, out=None, sel=None):
        spd, w = self.spd, self.w
        out = self.out if out is None else out
        sel = self.sel if sel is None else sel
        iq, q, bt, sl, kp, vp, ip = self.iq, self.q, self.bt, self.sl, self.kp[c], self.vp[c], self.ip[c]
        if self.f8:
            spd.mono_index_score_topk_fp8(iq, ip, bt, sl, w.k, T=w.T, out=sel, workspace=self.ws_topk)
            spd.mono_pa_decode_fp8(q, kp, vp, bt, sl, sel, w.scale, w.k_scale, w.v_scale, T=w.T, out=out,
                                   workspace=self.ws_pa)
        else:
            spd.mono_index_score_topk(iq, ip, bt, sl, w.k, T=w.T, out=sel, workspace=self.ws_topk)
            spd.mono_pa_decode_mxfp4(q, kp, vp, bt, sl, sel, w.scale, T=w.T, out=out, workspace=self.ws_pa)


def read_ceilings(spd, torch, dev, run, reps, grids=(256, 512, 1024, 2048)):
    """Read-bandwidth references over the workload's index pool, the pool
    copies rotated (cold reads): every byte in address order ("stream"), and
    the pages in block-table order with the index scan's lane pattern
    ("gather").  GB/s per grid size, from the kernel's mean duration."""
    w = run.w
    ids = np.concatenate([w.block_table[b, : -(-int(w.seq_lens[b]) // 128)] for b in range(w.B)]).astype(np.int32)
    ids_t = torch.from_numpy(ids).to(dev)
    sink = torch.empty(max(grids), dtype=torch.int32, device=dev)
    res = {}
    for mode, name in ((0, "stream"), (1, "gather")):
        n_pages = run.ip[0].shape[0] if mode == 0 else ids.size
        nbytes = n_pages * 8704
        kname = "read_stream_kernel" if mode == 0 else "read_gather_kernel"
        per = {}
        for grid in grids:
            for c in range(run.copies):  # warm-up
                spd.bench_read(run.ip[c], None if mode == 0 else ids_t, grid=grid, sink=sink)
            torch.cuda.synchronize(dev)
            with spd.KernelTimer(capacity=reps + 4) as kt:
                for r in range(reps):
                    spd.bench_read(run.ip[r % run.copies], None if mode == 0 else ids_t, grid=grid, sink=sink)
                torch.cuda.synchronize(dev)
            us = kt.mean_us[kname]
            per[str(grid)] = {"kernel_us_mean": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        res[name] = {"bytes_per_launch": nbytes, "by_grid": per,
                     "best_GBps": max(v["GBps"] for v in per.values())}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.timeline > 0:
        timeline(args)
        return

    import torch

    import sparse_paged_decode_amd as spd
    from workloads import workload

    spd.load_library()
    dev = torch.device("cuda:0")
    w = workload(args.workload, cache=args.cache)
    f8 = args.cache == "fp8"
    copies = max(1, args.copies)
    run = StepRunner(spd, torch, dev, w, copies)
    q, bt, sl, iq, kp, vp, ip = run.q, run.bt, run.sl, run.iq, run.kp, run.vp, run.ip
    sel = run.sel
    stream = torch.cuda.current_stream(dev)
    step, two_calls = run.step, run.two_calls

    for s in range(args.warmup):
        step(s % copies)
    torch.cuda.synchronize(dev)
    sel_np = sel.cpu().numpy() if w.sparse else None
    idx_bytes, kv_bytes = algorithmic_bytes(w, sel_np)
    bytes_step = idx_bytes + kv_bytes

    # Timed region: exactly K steps back to back, one event before the first
    # and one after the last, between synchronisations.
    K = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    ev0.record(stream)
    for s in range(K):
        step(s % copies)
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / K
    value = bytes_step / (ms_per_step * 1e-3) / 1e9

    # The spread of single steps: the same K steps again with an event pair
    # around each (the events add a little time between steps).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize(dev)
    for s in range(K):
        evs[s][0].record(stream)
        step(s % copies)
        evs[s][1].record(stream)
    torch.cuda.synchronize(dev)
    step_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])

    # Kernel-timing pass: the same K steps again, every kernel the library
    # launches bracketed by HIP events on its stream (the events add launch
    # gaps, so this pass is not the step time above); then the two-call
    # form of the step for reference.
    torch.cuda.synchronize(dev)
    with spd.KernelTimer(capacity=4 * K + 16) as kt:
        for s in range(K):
            step(s % copies)
        torch.cuda.synchronize(dev)
    two = {}
    if w.sparse and not args.skip_two_call:
        for s in range(args.warmup):
            two_calls(s % copies)
        torch.cuda.synchronize(dev)
        with spd.KernelTimer(capacity=4 * K + 16) as kt2:
            for s in range(K):
                two_calls(s % copies)
            torch.cuda.synchronize(dev)
        two = {name: round(us, 2) for name, us in kt2.mean_us.items()}

    # The same steps replayed from HIP graphs (one captured step per pool
    # copy), timed like the plain launches.
    graph_ms = graph_multi_ms = None
    if not args.skip_graph:
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        for s in range(args.warmup):
            graphs[s % copies].replay()
        torch.cuda.synchronize(dev)
        ge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ge[0].record(stream)
        for s in range(K):
            graphs[s % copies].replay()
        ge[1].record(stream)
        torch.cuda.synchronize(dev)
        graph_ms = ge[0].elapsed_time(ge[1]) / K
        # One graph holding one step per pool copy, replayed K / copies
        # times: the graph launch's own cost spread over several steps.
        gall = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gall):
            for c in range(copies):
                step(c)
        reps = max(1, K // copies)
        for _ in range(max(1, args.warmup // copies)):
            gall.replay()
        torch.cuda.synchronize(dev)
        ge[0].record(stream)
        for _ in range(reps):
            gall.replay()
        ge[1].record(stream)
        torch.cuda.synchronize(dev)
        graph_multi_ms = ge[0].elapsed_time(ge[1]) / (reps * copies)

    # Device error bits raised by any of the steps above (a bounded wait
    # that ran out, a bad page id or length): zero in a valid run.
    torch.cuda.synchronize(dev)
    device_errors = {name: int(spd.check_device_errors(wsx)) for name, wsx in
                     (("step", run.ws), ("index", run.ws_topk), ("attention", run.ws_pa))}

    # Clocks while the step runs back to back (sampled from sysfs).
    info, pci_dir = device_info(torch, dev)
    clocks = None
    if not args.skip_clocks:
        def run_steps(seconds):
            t_end = time.perf_counter() + seconds
            s = 0
            while time.perf_counter() < t_end:
                for _ in range(50):
                    step(s % copies)
                    s += 1
                torch.cuda.synchronize(dev)

        clocks = clocks_under_load(pci_dir, run_steps)

    # Roofline entry of the step kernel (on dense workloads the attention
    # kernel is the step).
    dom = ("sparse_decode_kernel" if w.sparse else "pa_decode_kernel").replace("_kernel", "_fp8_kernel" if f8 else "_kernel")
    dom_bytes = bytes_step
    dom_us = kt.mean_us[dom]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    # The cache insert (run last: it rewrites the decoded tokens' rows).
    ins = None
    if w.sparse and not f8 and not args.skip_insert:
        ins = time_insert(spd, torch, dev, w, kp, vp, ip, min(K, 100))
    cp = None
    if w.sparse and not f8 and not args.skip_cp:
        if 4 * w.k <= 8192:  # the merge takes at most 8192 candidates per query token
            cp = time_cp(spd, torch, dev, w, iq, ip[0], bt, sl, min(K, 50))
        else:
            cp = {"skipped": f"4 shards x top-{w.k} = {4 * w.k} candidates per query token; the merge takes 8192"}
    scan_variants = None
    if w.sparse and not f8 and not args.skip_scan_variants:
        scan_variants = time_scan_variants(spd, torch, dev, w, iq, ip[0], bt, sl, min(K, 50))
    ceilings = None
    if w.sparse and not f8 and not args.skip_ceilings:
        ceilings = read_ceilings(spd, torch, dev, run, min(K, 50))
    cpu = None
    if args.cpu_sample > 0:
        cpu = cpu_baseline(w, args.cpu_sample)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "B": w.B,
            "T": w.T,
            "context": int(w.seq_lens.max()) if w.T == 1 else [int(w.seq_lens.min()), int(w.seq_lens.max())],
            "k": w.k,
            "cache": w.cache,
            "pool_copies_rotated": copies,
        },
        "step_us": round(ms_per_step * 1e3, 2),
        "step_us_median": round(float(np.median(step_ms)) * 1e3, 2),
        "step_us_p90": round(float(np.percentile(step_ms, 90)) * 1e3, 2),
        "graph_step_us": round(graph_ms * 1e3, 2) if graph_ms is not None else None,
        "graph_step_us_steps_per_graph": {"1": round(graph_ms * 1e3, 2), str(copies): round(graph_multi_ms * 1e3, 2)}
        if graph_ms is not None else None,
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "bytes_per_step": {"index": idx_bytes, "kv": kv_bytes},
        "kernels_us_mean": {name: round(us, 2) for name, us in kt.mean_us.items()},
        "two_call_kernels_us_mean": two,
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": stored_traffic(dom, w.name),
            "algorithmic_bytes_per_launch": dom_bytes,
            "kernel_us_mean": round(dom_us, 3),
            "source_digest": kernel_digest(dom),
        },
        "device_errors": device_errors,
        "insert": ins,
        "cp_emulation": cp,
        "scan_mfma_vs_valu": scan_variants,
        "read_ceilings": ceilings,
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
        "device": info,
        "clocks_under_load": clocks,
        "hip": torch.version.hip,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
