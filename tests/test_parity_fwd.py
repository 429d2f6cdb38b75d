"""GPU forward parity against the CPU oracle (needs an MI355X).

Small seeded cases span several tiles, ragged tails, uncovered rows, r > H,
duplicate patterns, one-row segments, non-contiguous layouts and both merge
launch shapes (per residue class of n mod lcm(r), and per row); the
workload configurations run at full size (full-tensor where the oracle is
fast enough, sampled rows at 1M tokens).  Every call goes through the C ABI.
"""
import zlib

import numpy as np
import pytest

import oracle
from sparse_long_sequence_dilated_amd import dla, inputs
from tests.gpu_util import ORACLE_WORKERS, check_fwd, nan_like, nan_lse, to_device, to_host

pytestmark = pytest.mark.gpu

SMALL = [
    # (B, N, H, patterns, causal, dtype, layout)
    (2, 512, 3, ((128, 1), (256, 2), (512, 4)), True, "bf16", "bnhd"),
    (1, 1024, 2, ((1024, 1),), True, "bf16", "bnhd"),               # full attention, 4 tiles
    (1, 900, 2, ((300, 1), (900, 3)), True, "bf16", "bnhd"),         # L = 300: ragged tiles
    (2, 768, 3, ((768, 1),), False, "bf16", "bnhd"),
    (1, 900, 2, ((300, 1), (900, 3)), False, "bf16", "bnhd"),
    (1, 512, 3, ((256, 2),), True, "bf16", "bnhd"),                  # rows left uncovered
    (1, 1024, 2, ((64, 1), (256, 4), (1024, 16)), True, "bf16", "bnhd"),   # r > H
    (1, 512, 2, ((128, 2), (128, 2), (512, 1)), True, "bf16", "bnhd"),     # duplicate
    (1, 256, 3, ((4, 4), (64, 1)), True, "bf16", "bnhd"),            # one-row segments
    (2, 512, 3, ((128, 1), (512, 4)), True, "bf16", "bhnd"),         # [B,H,N,D] storage
    (3, 256, 1, ((256, 1), (256, 2)), True, "bf16", "bnhd"),
    (1, 600, 2, ((200, 1), (600, 2)), False, "f32", "bnhd"),
    (1, 600, 2, ((200, 1), (600, 2)), True, "f32", "bnhd"),
    (2, 512, 3, ((128, 1), (256, 2), (512, 4)), True, "f32", "bhnd"),
    (1, 256, 3, ((256, 4),), True, "f32", "bnhd"),                   # uncovered rows, fp32
    (1, 192, 2, ((3, 3), (192, 1)), False, "f32", "bnhd"),
    # N / lcm(r) < 32: the merge runs per row instead of per residue class
    (1, 256, 3, ((256, 1), (128, 16)), True, "bf16", "bnhd"),
    (2, 512, 2, ((512, 1), (256, 32)), False, "f32", "bnhd"),
    # a last segment cut short (w does not divide N, or w > N)
    (2, 1000, 3, ((256, 1), (512, 2), (2048, 4)), True, "bf16", "bnhd"),
    (1, 1000, 3, ((256, 1), (512, 2), (2048, 4)), False, "bf16", "bnhd"),
    (1, 602, 5, ((300, 4), (640, 1)), True, "bf16", "bhnd"),        # heads 2, 3: last segment empty
    (1, 1000, 2, ((4096, 1),), True, "bf16", "bnhd"),                # one segment shorter than w
    (2, 500, 3, ((128, 1), (256, 2), (1024, 4)), True, "f32", "bnhd"),
    (1, 500, 3, ((200, 4), (1024, 1)), False, "f32", "bnhd"),
    # residue-class merge where every class must be launched: two patterns of
    # rate 1, or none (rows left uncovered)
    (1, 2048, 3, ((128, 1), (256, 1), (512, 2), (1024, 4)), True, "bf16", "bnhd"),
    (1, 2048, 3, ((256, 2), (512, 4), (1024, 8)), True, "bf16", "bnhd"),
]


def _check_forward(q, k, v, pats, causal, scale, dtype, layout="bnhd", workers=1,
                   ref_dtype=np.float64):
    tq, tk, tv = (to_device(x, dtype, layout) for x in (q, k, v))
    o, lse = nan_like(tq), nan_lse(tq)
    dla.forward(tq, tk, tv, pats, causal, scale, out=o, lse=lse)
    import torch
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(q, k, v, pats, causal, scale, dtype=ref_dtype, workers=workers)
    return check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, dtype)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}N{c[1]}H{c[2]}-{c[5]}-{c[6]}-"
                         f"{'c' if c[4] else 'nc'}-{'_'.join(f'{w}x{r}' for w, r in c[3])}")
def test_forward_small_cases(case):
    B, N, H, pats, causal, dtype, layout = case
    print(f"case {case}", flush=True)
    q, k, v = inputs.random_case(zlib.crc32(repr(case).encode()) & 0xFFFF, B, N, H, dtype)
    _check_forward(q, k, v, pats, causal, 0.125, dtype, layout)


# The largest descriptor the ABI takes: 16 patterns.  The first mixes rates
# 3, 6 and 12 with powers of two (lcm 48 does not divide N: per-row merge)
# and cuts segments short; the second uses powers of two only (residue-class
# merge, only the classes another pattern keeps launched).
SIXTEEN = [
    (1, 1024, 3, ((64, 1), (128, 2), (256, 4), (512, 8), (1024, 16), (96, 3), (192, 6), (64, 2),
                  (128, 4), (256, 8), (32, 1), (512, 4), (1024, 2), (768, 3), (384, 12), (1024, 1))),
    (1, 2048, 2, ((64, 1), (128, 2), (256, 4), (512, 8), (1024, 16), (128, 4), (256, 2), (512, 16),
                  (1024, 8), (256, 8), (512, 2), (1024, 4), (128, 8), (256, 16), (512, 32), (1024, 32))),
]


@pytest.mark.parametrize("case", SIXTEEN, ids=["mixed_rates", "pow2_rates"])
def test_forward_sixteen_patterns(case):
    B, N, H, pats = case
    assert len(pats) == dla.MAX_PATTERNS
    print(f"case {case}", flush=True)
    q, k, v = inputs.random_case(zlib.crc32(repr(case).encode()) & 0xFFFF, B, N, H, "bf16")
    _check_forward(q, k, v, pats, True, 0.125, "bf16")


def test_forward_empty_batch():
    import torch
    q = torch.empty((0, 256, 2, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = dla.forward(q, q, q, [(64, 1)], True)
    assert o.shape == q.shape and lse.shape == (0, 2, 256)


def test_forward_rejects_bad_workspace():
    import torch
    q = torch.zeros((1, 256, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dla.DlaError) as ei:
        dla.forward(q, q, q, [(64, 1), (256, 4)], True,
                    workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert ei.value.code == dla.DLA_E_WORKSPACE


@pytest.mark.parametrize("N,pats", [(1000, ((256, 1), (512, 2), (2048, 4))), (602, ((300, 4), (640, 1)))])
def test_row_map_cut_short_segments_bit_exact(N, pats):
    for p, (w, r) in enumerate(pats):
        got = dla.row_map(pats, N, 5, p).cpu().numpy()
        for h in range(5):
            assert np.array_equal(got[h], oracle.row_map(N, w, r, h)), (N, p, h)


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4"])
def test_row_map_bit_exact(name):
    wl = inputs.WORKLOADS[name]
    for p, (w, r) in enumerate(wl.patterns):
        got = dla.row_map(wl.patterns, wl.N, wl.H, p).cpu().numpy()
        for h in range(wl.H):
            assert np.array_equal(got[h], oracle.row_map(wl.N, w, r, h)), (name, p, h)


@pytest.mark.parametrize("name", ["C1", "C2", "C3"])
def test_forward_workload_full_tensor(name):
    wl = inputs.WORKLOADS[name]
    print(wl.describe(), flush=True)
    q, k, v = inputs.workload_inputs(wl)
    ref_dtype = np.float64 if wl.dtype == "f32" else np.float32
    _check_forward(q, k, v, wl.patterns, wl.causal, wl.scale, wl.dtype,
                   workers=ORACLE_WORKERS, ref_dtype=ref_dtype)


def test_forward_c3_deterministic():
    import torch
    wl = inputs.WORKLOADS["C3"]
    q, k, v = (to_device(x, "bf16") for x in inputs.workload_inputs(wl))
    o1, l1 = dla.forward(q, k, v, wl.patterns, True)
    o2, l2 = dla.forward(q, k, v, wl.patterns, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.fixture(scope="module")
def c4_forward():
    """The 1M-token workload run once on the GPU into NaN-filled outputs:
    (q, k, v, o, lse) on the host, o as float32 [B, N, H, D]."""
    import torch
    wl = inputs.WORKLOADS["C4"]
    print(wl.describe(), flush=True)
    q, k, v = inputs.workload_inputs(wl)
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    o, lse = nan_like(tq), nan_lse(tq)
    dla.forward(tq, tk, tv, wl.patterns, True, out=o, lse=lse)
    torch.cuda.synchronize()
    del tq, tk, tv
    # every row is kept by the rate-1 pattern: nothing may stay unwritten,
    # whichever cache-sized schedule group its unit ran in
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    out = q, k, v, to_host(o), to_host(lse)
    del o, lse
    torch.cuda.empty_cache()
    return out


@pytest.mark.parametrize("h", range(12))
def test_forward_c4_full_tensor(c4_forward, h):
    """The 1M-token forward (34 cache-sized schedule groups) against the
    float32 oracle on every row, one head at a time (the oracle's buffers
    for all heads would need tens of GB)."""
    wl = inputs.WORKLOADS["C4"]
    q, k, v, o, lse = c4_forward
    sl = slice(h, h + 1)
    o_ref, lse_ref = oracle.forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], wl.patterns, True, wl.scale,
                                    dtype=np.float32, workers=ORACLE_WORKERS, heads=[h])
    check_fwd(o[:, :, h], lse[:, h], o_ref[:, :, 0], lse_ref[:, 0], "bf16", f"C4 head {h}:")


def test_forward_grouped_schedule_cut_short_full_tensor():
    """A problem large enough for several cache-sized schedule groups (each
    pattern's segment-heads split into runs, some units of the last run
    empty), with a cut-short last segment: every row of both batches and all
    heads against the float32 oracle, into NaN-filled outputs."""
    import torch
    B, N, H = 2, 65000, 12
    pats = ((2048, 1), (4096, 2), (16384, 8))
    q, k, v = inputs.random_case(6500, B, N, H, "bf16")
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    o, lse = nan_like(tq), nan_lse(tq)
    dla.forward(tq, tk, tv, pats, True, 0.125, out=o, lse=lse)
    torch.cuda.synchronize()
    del tq, tk, tv
    # every row is kept by the rate-1 pattern, so no entry may stay NaN
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    o_ref, l_ref = oracle.forward(q, k, v, pats, True, 0.125, dtype=np.float32, workers=ORACLE_WORKERS)
    check_fwd(to_host(o), to_host(lse), o_ref, l_ref, "bf16", f"grouped N={N}:")


def test_forward_long_segment_sampled_rows():
    """One segment of 65536 sparse rows (full causal attention over 64K rows:
    256 query units and 1024 key tiles per segment-head), plus a dilated
    pattern; sampled rows against the oracle one row at a time."""
    import torch
    B, N, H = 1, 65536, 2
    pats = ((65536, 1), (65536, 4))
    q, k, v = inputs.random_case(65536, B, N, H, "bf16")
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    o, lse = nan_like(tq), nan_lse(tq)
    dla.forward(tq, tk, tv, pats, True, 0.125, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    rows = np.array([0, 1, 63, 64, 255, 256, 4097, 32767, 32768, 65279, 65280, 65535])
    for h in (0, 1):
        o_ref, l_ref = oracle.forward_rows(q, k, v, pats, True, 0.125, 0, h, rows)
        idx = torch.from_numpy(rows).cuda()
        check_fwd(o[0, :, h][idx].float().cpu().numpy(), lse[0, h][idx].cpu().numpy(), o_ref, l_ref,
                  "bf16", f"long segment h={h}:")
