"""Host-side checks of the benchmark script: the one-GPU contract, the
algorithmic byte counts behind its HBM rooflines, and that the committed
traffic counters belong to the committed kernel sources."""
import json
import math
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from sparse_long_sequence_dilated_amd import inputs  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _row_by_row(family, wl):
    """The same byte counts, row by row over every (batch, row, head)."""
    D, total = wl.D, 0
    for _ in range(wl.B):
        for n in range(wl.N):
            for h in range(wl.H):
                kept = [p for p, (w, r) in enumerate(wl.patterns) if n % r == h % r]
                if len(kept) < 2:
                    continue
                if family == "bwd_finalize":
                    total += 3 * (len(kept) * D * 4 + D * 2)
                else:
                    total += (2 * D * 2 + 8) + (len(kept) - 1) * (D * 2 + 4)
    return total


@pytest.mark.parametrize("family", ["bwd_finalize", "combine"])
@pytest.mark.parametrize("pats", [[(256, 1), (512, 2), (1024, 4)],
                                  [(128, 1), (256, 2), (512, 4), (1024, 8), (1024, 16)],
                                  [(192, 1), (384, 3), (768, 6)]])
def test_hbm_byte_counts_match_a_row_by_row_count(family, pats):
    period = math.lcm(*[r for _, r in pats])
    wl = types.SimpleNamespace(B=2, N=16 * period * 4, H=5, D=64, patterns=pats)
    work, unit, bound = bench.family_work(family, wl, pairs=0)
    assert (unit, bound) == ("byte", "hbm")
    assert work == _row_by_row(family, wl)


def test_flop_counts_follow_the_pair_count():
    wl = inputs.WORKLOADS["C5"]
    assert bench.family_work("attn_fwd", wl, 1000) == (4 * 64 * 1000, "flop", "mfma")
    assert bench.family_work("attn_bwd", wl, 1000) == (10 * 64 * 1000, "flop", "mfma")


def test_traffic_counters_belong_to_the_committed_kernels():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    fams = [k for k in rec if not k.startswith("_")]
    assert set(fams) == set(bench.KERNEL_SOURCES)
    for fam in fams:
        assert rec[fam]["source_sha"] == bench.kernel_source_sha(fam), fam
        assert rec[fam]["bytes_per_launch"] > 0
