"""GPU parity of the LongNet attention layer (needs an MI355X).

The layer is Q, K, V = X W_q, X W_k, X W_v, A = DA(Q, K, V), Y = A W_o at the
model settings of the gptget.net summary of arXiv 2307.02486 (section
实验设计: 768 dimensions, 12 heads), with random weights.  Every call goes
through the C ABI (hipBLASLt projections, the library's attention); the
results are compared with the fp64 layer oracle on the same bf16 inputs.
At the 32K-token size every output and gradient is checked over the full
tensor, with the oracle's attention step in float32.
"""
import zlib

import numpy as np
import pytest

import oracle
from sparse_long_sequence_dilated_amd import dla, inputs
from tests.gpu_util import LSE_ABS, ORACLE_WORKERS, TOL, lse_abs, normwise, to_device, to_host

pytestmark = pytest.mark.gpu

H = 12
SCALE = 0.125

CASES = [
    # (B, N, patterns, causal)
    (2, 1024, ((256, 1), (512, 2), (1024, 4)), True),
    (1, 1000, ((512, 1), (1024, 2)), False),                    # cut-short segments
    (4, 2048, inputs.geometric_patterns(2048, 2, 5), True),     # 2K sequences, 32K pattern set;
                                                                # weight gradients in 4 row chunks
]


def _ids(c):
    return f"B{c[0]}N{c[1]}P{len(c[2])}-{'c' if c[3] else 'nc'}"


@pytest.fixture(scope="module")
def blas():
    b = dla.Blas()
    yield b
    b.close()


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_layer_forward_backward(case, blas):
    import torch
    B, N, pats, causal = case
    x, w_qkv, w_o, dy = inputs.layer_inputs(zlib.crc32(repr(case).encode()) & 0xFFFF, B, N, H)
    tx, twq, two, tdy = (to_device(t, "bf16") for t in (x, w_qkv, w_o, dy))
    y, qkv, attn, lse = dla.layer_forward(tx, twq, two, pats, blas, causal, SCALE)
    dx, dwq, dwo = dla.layer_backward(tx, twq, two, qkv, attn, lse, tdy, pats, blas, causal, SCALE)
    torch.cuda.synchronize()
    y_ref, saved = oracle.layer_forward(x, w_qkv, w_o, H, pats, causal, SCALE, workers=ORACLE_WORKERS)
    refs = oracle.layer_backward(x, w_qkv, w_o, saved, dy, pats, causal, SCALE, workers=ORACLE_WORKERS)
    checks = [("y", y, y_ref), ("attn", attn, saved[3]), ("lse", lse, saved[4])]
    checks += list(zip(("dx", "dw_qkv", "dw_o"), (dx, dwq, dwo), refs))
    for name, got, ref in checks:
        e = normwise(to_host(got), ref)
        print(f"{case[:2]} {name}: {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (name, e)
    la = lse_abs(to_host(lse), saved[4])
    print(f"{case[:2]} lse max abs {la:.3e} nats", flush=True)
    assert la <= LSE_ABS["bf16"]


def test_layer_32k_full_tensor(blas):
    """1 x 32768 tokens with the 32K pattern set: Y, A, LSE, dX, dW_qkv and dW_o
    over the full tensors against the layer oracle (float64 projections,
    float32 attention)."""
    import torch
    B, N = 1, 32768
    pats = inputs.geometric_patterns(2048, 2, 5)
    x, w_qkv, w_o, dy = inputs.layer_inputs(977, B, N, H)
    tx, twq, two, tdy = (to_device(t, "bf16") for t in (x, w_qkv, w_o, dy))
    y, qkv, attn, lse = dla.layer_forward(tx, twq, two, pats, blas, True, SCALE)
    dx, dwq, dwo = dla.layer_backward(tx, twq, two, qkv, attn, lse, tdy, pats, blas, True, SCALE)
    torch.cuda.synchronize()
    y_ref, saved = oracle.layer_forward(x, w_qkv, w_o, H, pats, True, SCALE, workers=ORACLE_WORKERS,
                                        attn_dtype=np.float32)
    refs = oracle.layer_backward(x, w_qkv, w_o, saved, dy, pats, True, SCALE, workers=ORACLE_WORKERS,
                                 attn_dtype=np.float32)
    checks = [("y", y, y_ref), ("attn", attn, saved[3]), ("lse", lse, saved[4])]
    checks += list(zip(("dx", "dw_qkv", "dw_o"), (dx, dwq, dwo), refs))
    for name, got, ref in checks:
        e = normwise(to_host(got), ref)
        print(f"32K {name}: {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (name, e)
    la = lse_abs(to_host(lse), saved[4])
    print(f"32K lse max abs {la:.3e} nats", flush=True)
    assert la <= LSE_ABS["bf16"]


def test_layer_rejects_bad_workspace(blas):
    import torch
    x, w_qkv, w_o, _ = inputs.layer_inputs(1, 1, 256, H)
    tx, twq, two = (to_device(t, "bf16") for t in (x, w_qkv, w_o))
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(dla.DlaError) as ei:
        dla.layer_forward(tx, twq, two, ((256, 1),), blas, True, SCALE, workspace=ws)
    assert ei.value.code == dla.DLA_E_WORKSPACE
