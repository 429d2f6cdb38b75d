"""Randomized GPU property tests (needs an MI355X).

Seeded random shapes and pattern sets, small enough for the brute-force
form: N in 1..300 (ragged, cut-short segments, w > N), 1..6 heads, 1..4
patterns with rates 1..8 (so r > H and uncovered rows occur), causal or not,
bf16 or fp32.  The forward is compared with the union-softmax brute force
(an independent formulation of the operator), and the bf16 backward with the
oracle's analytic gradients.  Outputs start filled with NaN, so an entry
the library fails to write is caught whatever memory held before.  Every
call goes through the C ABI.
"""
import numpy as np
import pytest

import oracle
from sparse_long_sequence_dilated_amd import dla, inputs
from tests.gpu_util import TOL, check_fwd, normwise, to_device, to_host

pytestmark = pytest.mark.gpu


def _case(seed):
    g = np.random.default_rng(seed)
    B = int(g.integers(1, 3))
    N = int(g.integers(1, 301))
    H = int(g.integers(1, 7))
    pats = []
    for _ in range(int(g.integers(1, 5))):
        r = int(g.choice([1, 2, 3, 4, 8]))
        L = int(g.integers(1, 80))
        pats.append((r * L, r))
    causal = bool(g.integers(0, 2))
    dtype = "f32" if seed % 4 == 3 else "bf16"
    return B, N, H, tuple(pats), causal, dtype


@pytest.mark.parametrize("seed", range(24))
def test_random_case_against_brute_force(seed):
    import torch
    B, N, H, pats, causal, dtype = _case(seed)
    print(f"seed {seed}: B={B} N={N} H={H} patterns={pats} causal={causal} {dtype}", flush=True)
    q, k, v, dout = inputs.random_case(9000 + seed, B, N, H, dtype, count=4)
    scale = 0.125
    tq, tk, tv, tdo = (to_device(x, dtype) for x in (q, k, v, dout))
    # outputs start as NaN, so an entry the library never writes cannot pass
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    dla.forward(tq, tk, tv, pats, causal, scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o_bf, lse_bf = oracle.brute_force_forward(q, k, v, pats, causal, scale)
    eo, el = check_fwd(to_host(o), to_host(lse), o_bf, lse_bf, dtype)
    if dtype != "bf16":
        return
    dq, dk, dv = (torch.full_like(tq, float("nan")) for _ in range(3))
    dla.backward(tq, tk, tv, o, lse, tdo, pats, causal, scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(q, k, v, pats, causal, scale)
    refs = oracle.backward(q, k, v, o_ref, lse_ref, dout, pats, causal, scale)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        e = normwise(to_host(got), ref)
        print(f"  {name} {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (name, e)


@pytest.mark.parametrize("seed", range(12))
def test_random_varlen_case(seed):
    """The same random cases (bf16) as batches of random lengths in 0..N."""
    import torch
    B, N, H, pats, causal, _ = _case(100 + seed)
    lens = [int(x) for x in np.random.default_rng(200 + seed).integers(0, N + 1, B)]
    print(f"seed {seed}: B={B} N={N} H={H} patterns={pats} causal={causal} lengths={lens}", flush=True)
    q, k, v, dout = inputs.random_case(9500 + seed, B, N, H, "bf16", count=4)
    tq, tk, tv, tdo = (to_device(x, "bf16") for x in (q, k, v, dout))
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    dla.forward_varlen(tq, tk, tv, lens, pats, causal, 0.125, out=o, lse=lse)
    dq, dk, dv = (torch.full_like(tq, float("nan")) for _ in range(3))
    dla.backward_varlen(tq, tk, tv, o, lse, tdo, lens, pats, causal, 0.125, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    o_bf, lse_bf = oracle.brute_force_forward(q, k, v, pats, causal, 0.125, lengths=lens)
    eo, el = check_fwd(to_host(o), to_host(lse), o_bf, lse_bf, "bf16")
    o_ref, lse_ref = oracle.forward(q, k, v, pats, causal, 0.125, lengths=lens)
    refs = oracle.backward(q, k, v, o_ref, lse_ref, dout, pats, causal, 0.125, lengths=lens)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        e = normwise(to_host(got), ref)
        print(f"  {name} {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (name, e)


@pytest.mark.parametrize("seed", range(8))
def test_random_fp8kv_case(seed):
    """Random cases with FP8 E4M3 keys and values: quantization bit-exact
    against the oracle, the forward against the brute force on the decoded
    keys and values."""
    import torch
    B, N, H, pats, causal, _ = _case(300 + seed)
    print(f"seed {seed}: B={B} N={N} H={H} patterns={pats} causal={causal}", flush=True)
    q, k, v = inputs.random_case(9700 + seed, B, N, H, "bf16")
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    k8, ks = dla.quantize_fp8(tk)
    v8, vs = dla.quantize_fp8(tv)
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    dla.forward_fp8kv(tq, k8, v8, ks, vs, pats, causal, 0.125, out=o, lse=lse)
    torch.cuda.synchronize()
    kc, ksc = oracle.quantize_per_head(k)
    vc, vsc = oracle.quantize_per_head(v)
    assert np.array_equal(k8.cpu().numpy(), kc) and np.array_equal(ks.cpu().numpy(), ksc)
    assert np.array_equal(v8.cpu().numpy(), vc) and np.array_equal(vs.cpu().numpy(), vsc)
    kd, vd = oracle.dequantize_per_head(kc, ksc), oracle.dequantize_per_head(vc, vsc)
    o_bf, lse_bf = oracle.brute_force_forward(q, kd, vd, pats, causal, 0.125)
    eo, el = check_fwd(to_host(o), to_host(lse), o_bf, lse_bf, "bf16")


def _large_case(seed):
    g = np.random.default_rng(seed)
    B = int(g.integers(1, 3))
    N = int(g.integers(300, 3001))
    H = int(g.integers(1, 5))
    pats = []
    for _ in range(int(g.integers(1, 4))):
        r = int(g.choice([1, 2, 4, 3]))
        L = int(g.integers(40, 700))
        pats.append((r * L, r))
    return B, N, H, tuple(pats), bool(g.integers(0, 2))


@pytest.mark.parametrize("seed", range(8))
def test_random_larger_case(seed):
    """Random cases of several 256-row query tiles and 64-row key tiles with
    ragged tails (N up to 3000, L up to 700), bf16 forward against the brute
    force and backward against the oracle."""
    import torch
    B, N, H, pats, causal = _large_case(400 + seed)
    print(f"seed {seed}: B={B} N={N} H={H} patterns={pats} causal={causal}", flush=True)
    q, k, v, dout = inputs.random_case(9900 + seed, B, N, H, "bf16", count=4)
    tq, tk, tv, tdo = (to_device(x, "bf16") for x in (q, k, v, dout))
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    dla.forward(tq, tk, tv, pats, causal, 0.125, out=o, lse=lse)
    dq, dk, dv = (torch.full_like(tq, float("nan")) for _ in range(3))
    dla.backward(tq, tk, tv, o, lse, tdo, pats, causal, 0.125, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    o_bf, lse_bf = oracle.brute_force_forward(q, k, v, pats, causal, 0.125)
    eo, el = check_fwd(to_host(o), to_host(lse), o_bf, lse_bf, "bf16")
    o_ref, lse_ref = oracle.forward(q, k, v, pats, causal, 0.125)
    refs = oracle.backward(q, k, v, o_ref, lse_ref, dout, pats, causal, 0.125)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        e = normwise(to_host(got), ref)
        print(f"  {name} {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (name, e)
