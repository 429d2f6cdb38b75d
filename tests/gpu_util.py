"""Helpers for GPU parity tests: host<->device marshalling and error norms."""
import os

import numpy as np

from sparse_long_sequence_dilated_amd import inputs

# Tolerances on the normwise relative error max|x - y| / max|y| against the
# oracle: fp32 paths 1e-5, bf16 paths (bf16 inputs, fp32 accumulation) 2e-2.
TOL = {"f32": 1e-5, "bf16": 2e-2}

ORACLE_WORKERS = max(1, min(16, os.cpu_count() or 1))


def to_device(x, dtype, layout="bnhd"):
    """Upload a float32 array holding exact `dtype` values; optionally as a [B,H,N,D]-stored view."""
    import torch
    if layout == "bhnd":
        x = np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))
    if dtype == "bf16":
        t = torch.from_numpy(inputs.bf16_bits(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.cuda()
    if layout == "bhnd":
        t = t.permute(0, 2, 1, 3)
    return t


def to_host(t):
    return t.float().cpu().numpy()


def normwise(x, ref):
    """max |x - ref| / max |ref| over finite reference entries; -inf must match exactly."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(x), fin), "non-finite pattern differs from the oracle"
    assert np.array_equal(x[~fin], ref[~fin]), "infinite entries differ from the oracle"
    if not fin.any():
        return 0.0
    den = np.abs(ref[fin]).max()
    return float(np.abs(x[fin] - ref[fin]).max() / (den if den > 0 else 1.0))


def nan_like(t):
    """A NaN-filled tensor with t's shape, strides and dtype: passed as an output
    buffer, any entry the library fails to write stays NaN and fails the check."""
    import torch
    return torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device).fill_(float("nan"))


def nan_lse(q):
    """A NaN-filled [B, H, N] float32 log-sum-exp buffer for q of shape [B, N, H, D]."""
    import torch
    B, N, H, _ = q.shape
    return torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
