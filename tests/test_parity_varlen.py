"""GPU parity of batches of different lengths (needs an MI355X).

Batch b is the sequence of its first lengths[b] rows; the rows after it are
padding (output 0, log-sum-exp -inf, zero gradients).  Segments are cut at a
batch's length as at the end of any sequence.  Compared with the oracle's
`lengths` path; every call goes through the C ABI.
"""
import zlib

import numpy as np
import pytest

import oracle
from sparse_long_sequence_dilated_amd import dla, inputs
from tests.gpu_util import TOL, check_fwd, normwise, to_device, to_host

pytestmark = pytest.mark.gpu

CASES = [
    # (N, H, patterns, causal, dtype, lengths)
    (1024, 3, ((256, 1), (512, 2), (1024, 4)), True, "bf16", (1024, 700, 0, 257)),
    (1024, 3, ((256, 1), (512, 2), (1024, 4)), False, "bf16", (1000, 64, 1024)),
    (768, 5, ((300, 4), (1024, 1)), True, "bf16", (602, 768, 1)),
    (512, 2, ((512, 1),), True, "bf16", (300, 512)),                 # one pattern, no merge pass
    (600, 3, ((200, 1), (600, 2)), True, "f32", (600, 333, 0)),
    (600, 3, ((200, 1), (600, 2)), False, "f32", (17, 600)),
]


def _ids(c):
    return f"N{c[0]}H{c[1]}-{c[4]}-{'c' if c[3] else 'nc'}-L{'_'.join(map(str, c[5]))}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_varlen_forward_and_backward(case):
    import torch
    N, H, pats, causal, dtype, lens = case
    B = len(lens)
    q, k, v, dout = inputs.random_case(zlib.crc32(repr(case).encode()) & 0xFFFF, B, N, H, dtype, count=4)
    tq, tk, tv, tdo = (to_device(x, dtype) for x in (q, k, v, dout))
    # outputs start as NaN, so an entry the library never writes cannot pass
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    dla.forward_varlen(tq, tk, tv, lens, pats, causal, 0.125, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(q, k, v, pats, causal, 0.125, lengths=lens)
    eo, el = check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, dtype)
    for b, n_b in enumerate(lens):
        assert torch.all(o[b, n_b:] == 0) and torch.all(lse[b, :, n_b:] == float("-inf"))
    if dtype != "bf16":
        return
    dq, dk, dv = (torch.full_like(tq, float("nan")) for _ in range(3))
    dla.backward_varlen(tq, tk, tv, o, lse, tdo, lens, pats, causal, 0.125, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    refs = oracle.backward(q, k, v, o_ref, lse_ref, dout, pats, causal, 0.125, lengths=lens)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        e = normwise(to_host(got), ref)
        print(f"{case} {name}: {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (name, e)
        for b, n_b in enumerate(lens):
            assert torch.all(got[b, n_b:] == 0)


def test_varlen_lengths_are_clamped():
    import torch
    pats = ((256, 1), (512, 2))
    q, k, v = inputs.random_case(5, 3, 512, 2, "bf16")
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    o1, l1 = dla.forward_varlen(tq, tk, tv, (512 + 100, -5, 512), pats, True, 0.125)
    o2, l2 = dla.forward_varlen(tq, tk, tv, (512, 0, 512), pats, True, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_varlen_full_lengths_equal_the_plain_call():
    import torch
    pats = ((256, 1), (512, 2), (1024, 4))
    q, k, v, dout = inputs.random_case(9, 2, 1024, 3, "bf16", count=4)
    tq, tk, tv, tdo = (to_device(x, "bf16") for x in (q, k, v, dout))
    o1, l1 = dla.forward_varlen(tq, tk, tv, (1024, 1024), pats, True, 0.125)
    o2, l2 = dla.forward(tq, tk, tv, pats, True, 0.125)
    g1 = dla.backward_varlen(tq, tk, tv, o1, l1, tdo, (1024, 1024), pats, True, 0.125)
    g2 = dla.backward(tq, tk, tv, o2, l2, tdo, pats, True, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
