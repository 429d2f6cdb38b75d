"""GPU parity of 8-bit keys and values (needs an MI355X).

dla_quantize_fp8 must give the oracle's codes and scales bit for bit (the
same fp32 amax, 448 / amax and x * inv, then round-to-nearest-even to E4M3).
dla_forward_fp8kv is compared with the fp64 oracle forward on the decoded
keys and values, code * scale, at the bf16 tolerance; at the 32K-token size
over the full tensor (float32 oracle).  Every call goes through the C ABI.
"""
import zlib

import numpy as np
import pytest

import oracle
from sparse_long_sequence_dilated_amd import dla, inputs
from tests.gpu_util import ORACLE_WORKERS, check_fwd, to_device, to_host

pytestmark = pytest.mark.gpu


def _seed(case):
    return zlib.crc32(repr(case).encode()) & 0xFFFF


@pytest.mark.parametrize("layout", ["bnhd", "bhnd"])
def test_quantize_matches_oracle_bit_exact(layout):
    x, = inputs.draw((2, 700, 3, 64), 5, 1, "bf16")
    x[0, :, 1] = 0.0                            # an all-zero head: codes 0, scale 1
    x[1, :, 2] *= 2.0 ** -12                    # small values: subnormal codes
    x[1, 5, 0, 7] = 300.0                       # one outlier sets its head's scale
    t = to_device(x, "bf16", layout)
    codes, scale = dla.quantize_fp8(t)
    ref_codes, ref_scale = oracle.quantize_per_head(x)
    got = codes.cpu().numpy()
    assert np.array_equal(scale.cpu().numpy(), ref_scale)
    assert np.array_equal(got, ref_codes), int((got != ref_codes).sum())


def test_quantize_empty_sequence_gives_unit_scales():
    import torch
    x = torch.empty((2, 0, 3, 64), dtype=torch.bfloat16, device="cuda")
    _, scale = dla.quantize_fp8(x)
    assert torch.all(scale == 1.0)


CASES = [
    # (B, N, H, patterns, causal)
    (2, 1024, 3, ((256, 1), (512, 2), (1024, 4)), True),
    (1, 1024, 3, ((256, 1), (512, 2), (1024, 4)), False),
    (1, 1000, 5, ((300, 4), (1024, 1)), True),                # cut-short segments, r > H offsets
    (1, 512, 2, ((512, 1),), True),                            # one pattern, no merge
    (1, 4096, 12, inputs.geometric_patterns(2048, 2, 2), True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}N{c[1]}H{c[2]}P{len(c[3])}-{'c' if c[4] else 'nc'}")
def test_forward_fp8kv_matches_oracle(case):
    import torch
    B, N, H, pats, causal = case
    q, k, v = inputs.random_case(_seed(case), B, N, H, "bf16")
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    k8, ks = dla.quantize_fp8(tk)
    v8, vs = dla.quantize_fp8(tv)
    o, lse = dla.forward_fp8kv(tq, k8, v8, ks, vs, pats, causal, 0.125)
    torch.cuda.synchronize()
    kc, ksc = oracle.quantize_per_head(k)
    vc, vsc = oracle.quantize_per_head(v)
    kd, vd = oracle.dequantize_per_head(kc, ksc), oracle.dequantize_per_head(vc, vsc)
    o_ref, lse_ref = oracle.forward(q, kd, vd, pats, causal, 0.125, workers=ORACLE_WORKERS)
    eo, el = check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, "bf16")


def test_forward_fp8kv_32k_full_tensor():
    """The 32K-token workload (B=1, H=12, w = 2048 2^i, r = 2^i, i = 0..4) with
    8-bit keys and values: codes and scales bit-exact, then every output
    row and LSE entry against the float32 oracle on the decoded keys and
    values, into NaN-filled outputs so that a row no unit writes cannot pass."""
    import torch
    wl = inputs.WORKLOADS["C3"]
    q, k, v = inputs.workload_inputs(wl)
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    k8, ks = dla.quantize_fp8(tk)
    v8, vs = dla.quantize_fp8(tv)
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((wl.B, wl.H, wl.N), float("nan"), dtype=torch.float32, device="cuda")
    dla.forward_fp8kv(tq, k8, v8, ks, vs, wl.patterns, wl.causal, wl.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    kc, ksc = oracle.quantize_per_head(k)
    assert np.array_equal(k8.cpu().numpy(), kc) and np.array_equal(ks.cpu().numpy(), ksc)
    vc, vsc = oracle.quantize_per_head(v)
    assert np.array_equal(v8.cpu().numpy(), vc) and np.array_equal(vs.cpu().numpy(), vsc)
    kd, vd = oracle.dequantize_per_head(kc, ksc), oracle.dequantize_per_head(vc, vsc)
    o_ref, lse_ref = oracle.forward(q, kd, vd, wl.patterns, wl.causal, wl.scale, dtype=np.float32,
                                    workers=ORACLE_WORKERS)
    check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, "bf16", tag="C3 fp8")


def test_forward_fp8kv_rejects_fp32():
    import torch
    q = torch.zeros((1, 256, 2, 64), dtype=torch.float32, device="cuda")
    k8 = torch.zeros(q.shape, dtype=torch.uint8, device="cuda")
    s = torch.ones((1, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(dla.DlaError) as ei:
        dla.forward_fp8kv(q, k8, k8, s, s, ((256, 1),), True, 0.125)
    assert ei.value.code == dla.DLA_E_UNSUPPORTED
