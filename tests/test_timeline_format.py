"""The timeline printer of bench.py on synthetic trace records (CPU only).

Records follow include/mono_trace.h: item record t holds stamps (100 MHz
ticks) at words 0 (start), 1 (end), 2..30 (phases) and the kind word 31;
workgroup record w holds its kernel entry (0) and exit (1).
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _records():
    it = np.zeros((8192, 32), dtype=np.int64)
    gr = np.zeros((4096, 32), dtype=np.int64)
    t0 = 1_000_000
    for w in range(4):
        gr[w, 0] = t0 + 10 * w
        gr[w, 1] = t0 + 5000
    # four chunk-local items (kind 1 with stamp 4): the first two workgroups
    # of the grid scan for 20 us, the other two for 24 us; each later phase
    # takes 1 us, the merge (stamp 16) only in item 3.
    for t in range(4):
        it[t, 31] = (1 << 24) | t
        it[t, 0] = t0 + 100
        scan = 2000 if t < 2 else 2400
        it[t, 2] = it[t, 0] + scan
        for k in range(3, 16):
            it[t, k] = it[t, k - 1] + 100
        if t == 3:
            it[t, 16] = it[t, 15] + 100
        it[t, 1] = it[t, 15] + 200
    # two attention items (kind 3)
    for t in (4, 5):
        it[t, 31] = (3 << 24) | (t - 4)
        it[t, 0] = t0 + 300
        for k in range(10, 16):
            it[t, k] = it[t, 0] + 50 * (k - 9)
        it[t, 1] = it[t, 15] + 10
    return it, gr


def test_print_timeline(capsys):
    it, gr = _records()
    bench.print_timeline(0, it, gr)
    out = capsys.readouterr().out
    assert "4 workgroups enter over 0.30 us" in out
    assert "the last leaves the item loop at 50.00 us" in out
    assert "chunk-local chunk: 4 items" in out and "attention split: 2 items" in out
    lines = {l.split("  ")[0].strip(): l for l in out.splitlines() if l.startswith("    ") and "  " in l.strip()}
    scan = [l for l in out.splitlines() if l.strip().startswith("scan and histogram flush done")][0].split()
    # p50 of 21 / 21 / 25 / 25 us after the first entry; step p50 22 us (20 and 24 us)
    assert scan[-6:] == ["4", "21.00", "23.00", "25.00", "25.00", "22.00"], scan
    merged = [l for l in out.splitlines() if "attention: merged" in l][0].split()
    assert merged[-6] == "1" and merged[-1] == "1.00", merged  # one item, 1 us after its arrival
    end = [l for l in out.splitlines() if l.strip().startswith("end")]
    assert end[0].split()[-1] == "2.00"  # chunk items: 2 us after their last stamp (arrival), p50
    slot = [l for l in out.splitlines() if "the first workgroup of each CU" in l][0]
    assert "20.00 us for tickets below 2" in slot and "24.00 us for tickets 2..3" in slot
    assert lines  # the table rows parse
