"""Helpers for GPU parity tests: host<->device marshalling and error norms."""
import os

import numpy as np

from sparse_long_sequence_dilated_amd import inputs

# Tolerances on the normwise relative error max|x - y| / max|y| against the
# oracle: fp32 paths 1e-5, bf16 paths (bf16 inputs, fp32 accumulation) 2e-2.
TOL = {"f32": 1e-5, "bf16": 2e-2}
# The log-sum-exp is also bounded entry by entry in absolute terms (nats):
# the merge weights exp(LSE_p - LSE) and the backward's P = exp(S - LSE) move
# by a factor exp(e) ~ 1 + e for an LSE error of e, so the same numbers bound
# it as a relative error on those weights.  (A normwise bound alone would let
# e reach TOL * max|LSE|, about 0.17 nats at max|LSE| ~ 8.5.)  For fp32 the
# bound is relative to the entry, 1e-5 * max(1, |LSE|), the fp32 tolerance
# itself: fp32 rounding of the log2-domain scores grows with their size.
LSE_ABS = {"f32": 1e-5, "bf16": 2e-2}

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


def elementwise(x, ref):
    """max |x - ref| / max(|ref|, 1e-3 * max|ref|) over finite reference
    entries: the entry-by-entry relative error, with a floor that keeps
    entries near zero from dominating (reported beside the normwise error)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    if not fin.any():
        return 0.0
    r = np.abs(ref[fin])
    floor = 1e-3 * r.max()
    if floor == 0:
        return float(np.abs(x[fin]).max())
    return float((np.abs(x[fin] - ref[fin]) / np.maximum(r, floor)).max())


def lse_abs(x, ref):
    """max |x - ref| in nats over finite reference entries (-inf must match exactly)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(x), fin), "non-finite pattern differs from the oracle"
    assert np.array_equal(x[~fin], ref[~fin]), "infinite entries differ from the oracle"
    return float(np.abs(x[fin] - ref[fin]).max()) if fin.any() else 0.0


def lse_rel(x, ref):
    """max |x - ref| / max(1, |ref|) over finite reference entries."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    lse_abs(x, ref)                                   # the same checks of non-finite entries
    fin = np.isfinite(ref)
    if not fin.any():
        return 0.0
    return float((np.abs(x[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))).max())


def check_fwd(o, lse, o_ref, lse_ref, dtype, tag="", lse_bound=None):
    """Forward outputs against the oracle: O and LSE normwise within TOL, LSE
    entry by entry within LSE_ABS nats (bf16; `lse_bound` overrides it) or
    within 1e-5 * max(1, |LSE|) (fp32); prints the elementwise error too.
    Returns (O normwise, LSE normwise)."""
    o = np.asarray(o)
    lse = np.asarray(lse)
    eo, el = normwise(o, o_ref), normwise(lse, lse_ref)
    la = lse_abs(lse, lse_ref)
    print(f"{tag} O normwise {eo:.3e} elementwise {elementwise(o, o_ref):.3e}; "
          f"LSE normwise {el:.3e} max abs {la:.3e} nats", flush=True)
    assert eo <= TOL[dtype], f"{tag} O error {eo}"
    assert el <= TOL[dtype], f"{tag} LSE error {el}"
    if dtype == "f32":
        lr = lse_rel(lse, lse_ref)
        assert lr <= LSE_ABS[dtype], f"{tag} LSE error {lr} relative to max(1, |LSE|)"
    else:
        bound = LSE_ABS[dtype] if lse_bound is None else lse_bound
        assert la <= bound, f"{tag} LSE absolute error {la} nats (bound {bound})"
    return eo, el


def check_grads(got, refs, tag=""):
    """bf16 gradients (dq, dk, dv) against the oracle: normwise within
    TOL['bf16'], elementwise error printed.  Returns {name: normwise}."""
    errs = {}
    for name, g, ref in zip(("dq", "dk", "dv"), got, refs):
        g = np.asarray(g)
        errs[name] = normwise(g, ref)
        print(f"{tag} {name} normwise {errs[name]:.3e} elementwise {elementwise(g, ref):.3e}", flush=True)
        assert errs[name] <= TOL["bf16"], (tag, name, errs[name])
    return errs


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
