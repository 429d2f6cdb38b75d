"""GPU parity of the softmax offset paths (needs an MI355X).

The bf16 forward starts a wave's running offset at the exact row maximum of
its first 32 keys and raises it only when a lane's partial row sum passes
2^16.  Unit-variance inputs at scale 1/8 almost never raise it; the cases
here do, often and by large steps: logits several times larger, logits that
grow along the sequence, and a first key block far below the rest.  They
also hold the forward's rounding to account at logit sizes where an extra
rounding of the scores would show.  Outputs against the float64 oracle on the same bf16 inputs,
the bf16 backward against its analytic gradients, through the C ABI.
"""
import numpy as np
import pytest

import oracle
from sparse_long_sequence_dilated_amd import dla, inputs
from tests.gpu_util import check_fwd, check_grads, nan_like, nan_lse, to_device, to_host

pytestmark = pytest.mark.gpu

PATS = ((256, 1), (512, 2), (1024, 4))


def _run(q, k, v, dout, pats, causal, scale, dtype, tag):
    import torch
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = nan_like(tq), nan_lse(tq)
    dla.forward(tq, tk, tv, pats, causal, scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(q, k, v, pats, causal, scale)
    check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, dtype, tag)
    if dtype != "bf16":
        return
    tdo = to_device(dout, dtype)
    dq, dk, dv = (nan_like(tq) for _ in range(3))
    dla.backward(tq, tk, tv, o, lse, tdo, pats, causal, scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    refs = oracle.backward(q, k, v, o_ref, lse_ref, dout, pats, causal, scale)
    check_grads([to_host(t) for t in (dq, dk, dv)], refs, tag)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [0.5, 1.0])
def test_large_logits(scale, dtype):
    """Logits with a standard deviation of 4 and 8 (log2 units 5.8 and 11.5):
    most waves start from the exact maximum, and later key blocks raise it."""
    q, k, v, dout = inputs.random_case(4100, 1, 1024, 2, dtype, count=4)
    _run(q, k, v, dout, PATS, True, scale, dtype, f"scale {scale} {dtype}:")


def test_growing_logits():
    """Keys scaled up along the sequence (1x to 6x): a wave starts on the
    offset-0 path and the row sums of later blocks pass 2^16, so the offset
    is raised and O and l rescaled, several times per row."""
    q, k, v, dout = inputs.random_case(4200, 2, 1024, 2, "bf16", count=4)
    ramp = 1.0 + 5.0 * np.arange(1024, dtype=np.float32) / 1023.0
    k = inputs.round_to_bf16(k * ramp[None, :, None, None])
    _run(q, k, v, dout, PATS, True, 0.25, "bf16", "growing logits:")


def test_first_keys_far_below():
    """Every query close to one direction u and the first 64 keys at -8 u: the
    first key block's row maxima lie far below -64 (log2 units), so a wave
    starts from the exact maximum and the next blocks raise it by about 100."""
    g = np.random.default_rng(4300)
    N, H = 1024, 2
    u = g.standard_normal(64).astype(np.float32)
    u *= 3.0 / np.linalg.norm(u)
    q = u[None, None, None, :] + 0.3 * g.standard_normal((1, N, H, 64)).astype(np.float32)
    k = g.standard_normal((1, N, H, 64)).astype(np.float32)
    k[:, :64] = -8.0 * u[None, None, :] + 0.1 * g.standard_normal((1, 64, H, 64)).astype(np.float32)
    v = g.standard_normal((1, N, H, 64)).astype(np.float32)
    dout = g.standard_normal((1, N, H, 64)).astype(np.float32)
    q, k, v, dout = (inputs.round_to_bf16(x) for x in (q, k, v, dout))
    _run(q, k, v, dout, ((1024, 1), (1024, 2)), True, 0.7, "bf16", "first keys far below:")
