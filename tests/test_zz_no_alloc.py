"""dla_forward_noalloc (the forward on the library's static scratch) against
dla_forward (the same kernels on a caller's workspace), through the C ABI.

Two calls in a row, the second on a smaller problem, so that the scratch
holds the first call's partial results when the second runs; both must match
dla_forward bit for bit (same kernels, same order of arithmetic) and the
oracle within the bf16 tolerance.  A problem whose workspace exceeds the
scratch is refused before anything is enqueued.
"""
import numpy as np
import pytest

import oracle
from sparse_long_sequence_dilated_amd import dla, inputs
from tests.gpu_util import check_fwd, nan_like, nan_lse, to_device, to_host

pytestmark = pytest.mark.gpu


def _pair(seed, B, N, H, pats):
    import torch
    q, k, v = inputs.random_case(seed, B, N, H, "bf16")
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    o_ref, lse_ref = dla.forward(tq, tk, tv, pats, True, 0.125)
    o, lse = nan_like(tq), nan_lse(tq)
    dla.forward_noalloc(tq, tk, tv, pats, True, 0.125, out=o, lse=lse)
    torch.cuda.synchronize()
    return (q, k, v), (o, lse), (o_ref, lse_ref)


def test_noalloc_forward_matches_forward_twice_shrinking():
    import torch
    # C3's pattern set at B = 1, N = 32768 (41 MB of partials), then a
    # smaller problem with a different pattern set: the second call finds the
    # first call's partials in the scratch.
    cases = [(3301, 1, 32768, 12, inputs.WORKLOADS["C3"].patterns),
             (3302, 2, 3000, 5, ((256, 1), (512, 2), (1536, 4), (3000, 3)))]
    for seed, B, N, H, pats in cases:
        ws_f, _ = dla.plan_check(pats, True, 0.125, B, N, H)
        assert 0 < ws_f <= dla.NOALLOC_SCRATCH_BYTES
        print(f"case B={B} N={N} H={H} patterns={pats}: workspace {ws_f} bytes", flush=True)
        (q, k, v), (o, lse), (o_ref, lse_ref) = _pair(seed, B, N, H, pats)
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        if N <= 4096:
            ro, rl = oracle.forward(q, k, v, pats, True, 0.125)
            check_fwd(to_host(o), to_host(lse), ro, rl, "bf16", f"noalloc N={N}:")


def test_noalloc_forward_rejects_a_workspace_beyond_the_scratch():
    import torch
    pats = inputs.WORKLOADS["C3"].patterns
    B, N, H = 4, 32768, 12          # 164 MB of partials
    ws_f, _ = dla.plan_check(pats, True, 0.125, B, N, H)
    assert ws_f > dla.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, N, H, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    with pytest.raises(dla.DlaError) as ei:
        dla.forward_noalloc(q, q, q, pats, True, 0.125, out=o)
    assert ei.value.code == dla.DLA_E_WORKSPACE
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)       # nothing was enqueued


def test_noalloc_forward_one_pattern_needs_no_scratch():
    """A single pattern writes o and lse directly (no partials)."""
    import torch
    (q, k, v), (o, lse), (o_ref, lse_ref) = _pair(3303, 1, 1000, 3, ((256, 1),))
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    ro, rl = oracle.forward(q, k, v, ((256, 1),), True, 0.125)
    check_fwd(to_host(o), to_host(lse), ro, rl, "bf16", "noalloc one pattern:")
    assert np.isfinite(to_host(lse)).all()
