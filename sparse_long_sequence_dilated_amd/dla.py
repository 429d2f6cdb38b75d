"""ctypes binding of libdla (include/dla.h): argument marshalling only.

PyTorch provides device memory and the current HIP stream; every step of the
computation runs in libdla's kernels.  The library must have been built
(``python -m sparse_long_sequence_dilated_amd.build``); loading fails loudly
otherwise, and there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdla.so")

DLA_OK = 0
DLA_E_INVALID = -1
DLA_E_UNSUPPORTED = -2
DLA_E_WORKSPACE = -3
DLA_E_HIP = -4
DLA_F32 = 0
DLA_BF16 = 1
MAX_PATTERNS = 16
HEAD_DIM = 64

EXPORTS = ("dla_plan_check", "dla_forward", "dla_backward", "dla_row_map", "dla_pair_count",
           "dla_plan_check_shard", "dla_pair_count_shard", "dla_shard_gather", "dla_forward_shard",
           "dla_backward_shard", "dla_shard_finish", "dla_forward_varlen", "dla_backward_varlen",
           "dla_pair_count_varlen", "dla_blas_create", "dla_blas_destroy", "dla_layer_plan_check",
           "dla_layer_forward", "dla_layer_backward", "dla_quantize_fp8", "dla_forward_fp8kv",
           "dla_forward_noalloc", "dla_timing_enable", "dla_timing_collect", "dla_strerror",
           "dla_last_error")


class DlaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libdla error {code}: {msg}")
        self.code = code


class Pattern(ctypes.Structure):
    _fields_ = [("w", ctypes.c_int32), ("r", ctypes.c_int32)]


class Desc(ctypes.Structure):
    _fields_ = [("num_patterns", ctypes.c_int32), ("patterns", ctypes.POINTER(Pattern)),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_float)]


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("N", ctypes.c_int64), ("H", ctypes.c_int64),
                ("D", ctypes.c_int64), ("dtype", ctypes.c_int32), ("stride_b", ctypes.c_int64),
                ("stride_n", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class Shard(ctypes.Structure):
    _fields_ = [("total_rows", ctypes.c_int64), ("shard_start", ctypes.c_int64)]


_lib = None


def lib():
    """Load libdla.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_long_sequence_dilated_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    pd, ps = ctypes.POINTER(Desc), ctypes.POINTER(Shape)
    L.dla_plan_check.argtypes = [pd, ps, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.dla_forward.argtypes = [pd, ps, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dla_forward_noalloc.argtypes = [pd, ps, vp, vp, vp, vp, vp, vp]
    L.dla_backward.argtypes = [pd, ps, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dla_row_map.argtypes = [pd, i64, i32, i32, vp, vp]
    L.dla_pair_count.argtypes = [pd, ps, ctypes.POINTER(i64)]
    psh = ctypes.POINTER(Shard)
    L.dla_plan_check_shard.argtypes = [pd, ps, psh, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.dla_pair_count_shard.argtypes = [pd, ps, psh, ctypes.POINTER(i64)]
    L.dla_shard_gather.argtypes = [pd, ps, psh, i32, vp, vp, vp]
    L.dla_forward_shard.argtypes = [pd, ps, psh, vp, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                    vp, vp, vp, sz, vp]
    pvp = ctypes.POINTER(vp)
    L.dla_backward_shard.argtypes = [pd, ps, psh, vp, vp, vp, vp, vp, vp, pvp, pvp, vp, vp, vp, pvp, pvp,
                                     vp, sz, vp]
    L.dla_shard_finish.argtypes = [pd, ps, psh, pvp, pvp, vp, vp, vp, sz, vp]
    L.dla_forward_varlen.argtypes = [pd, ps, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dla_backward_varlen.argtypes = [pd, ps, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dla_pair_count_varlen.argtypes = [pd, ps, ctypes.POINTER(i32), ctypes.POINTER(i64)]
    L.dla_quantize_fp8.argtypes = [ps, vp, vp, vp, vp]
    L.dla_forward_fp8kv.argtypes = [pd, ps, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dla_blas_create.argtypes = [ctypes.POINTER(vp)]
    L.dla_blas_destroy.argtypes = [vp]
    L.dla_layer_plan_check.argtypes = [pd, i64, i64, i64, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.dla_layer_forward.argtypes = [pd, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dla_layer_backward.argtypes = [pd, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     sz, vp]
    L.dla_timing_enable.argtypes = [ctypes.c_int]
    L.dla_timing_enable.restype = ctypes.c_int
    L.dla_timing_collect.argtypes = [ctypes.c_char_p, ctypes.POINTER(i64),
                                     ctypes.POINTER(ctypes.c_double)]
    L.dla_timing_collect.restype = ctypes.c_int
    L.dla_strerror.argtypes = [ctypes.c_int]
    L.dla_strerror.restype = ctypes.c_char_p
    L.dla_last_error.argtypes = []
    L.dla_last_error.restype = ctypes.c_char_p
    for name in ("dla_plan_check", "dla_forward", "dla_backward", "dla_row_map", "dla_pair_count",
                 "dla_plan_check_shard", "dla_pair_count_shard", "dla_shard_gather",
                 "dla_forward_shard", "dla_backward_shard", "dla_shard_finish",
                 "dla_forward_varlen", "dla_backward_varlen", "dla_pair_count_varlen",
                 "dla_blas_create", "dla_blas_destroy", "dla_layer_plan_check", "dla_layer_forward",
                 "dla_layer_backward", "dla_quantize_fp8", "dla_forward_fp8kv", "dla_forward_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int):
    if rc != DLA_OK:
        raise DlaError(rc, lib().dla_last_error().decode() or lib().dla_strerror(rc).decode())


def make_desc(patterns, causal: bool, scale: float):
    arr = (Pattern * max(1, len(patterns)))(*[Pattern(int(w), int(r)) for w, r in patterns])
    d = Desc(len(patterns), ctypes.cast(arr, ctypes.POINTER(Pattern)), int(bool(causal)),
             float(scale))
    d._keep = arr  # keep the pattern array alive with the descriptor
    return d


def make_shape(B, N, H, D, dtype, strides=None):
    if strides is None:
        strides = (N * H * D, H * D, D)
    return Shape(B, N, H, D, dtype, *strides)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return DLA_F32
    if t.dtype == torch.bfloat16:
        return DLA_BF16
    raise DlaError(DLA_E_UNSUPPORTED, f"dtype {t.dtype} is neither float32 nor bfloat16")


def _shape_of(t):
    if t.dim() != 4:
        raise DlaError(DLA_E_INVALID, "tensors must be [B, N, H, D]")
    if t.stride(3) != 1:
        raise DlaError(DLA_E_INVALID, "the last dimension must be contiguous")
    B, N, H, D = t.shape
    return make_shape(B, N, H, D, _dtype_code(t), (t.stride(0), t.stride(1), t.stride(2)))


def _same_layout(ref, *ts):
    for t in ts:
        if t.shape != ref.shape or t.stride() != ref.stride() or t.dtype != ref.dtype:
            raise DlaError(DLA_E_INVALID, "q, k, v, o (and gradients) need one shape, stride and dtype")
        if t.device != ref.device:
            raise DlaError(DLA_E_INVALID, "all tensors must be on one device")


def _check_lse(lse, q):
    """lse must be a contiguous float32 [B, H, N] tensor on q's device."""
    import torch
    B, N, H, _ = q.shape
    if (not isinstance(lse, torch.Tensor) or lse.shape != (B, H, N) or not lse.is_contiguous()
            or lse.dtype != torch.float32 or lse.device != q.device):
        raise DlaError(DLA_E_INVALID, "lse must be a contiguous float32 [B, H, N] tensor on q's device")


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def plan_check(patterns, causal, scale, B, N, H, D=HEAD_DIM, dtype=DLA_BF16, strides=None):
    """Return (ws_fwd_bytes, ws_bwd_bytes); raises DlaError on an invalid problem."""
    d = make_desc(patterns, causal, scale)
    s = make_shape(B, N, H, D, dtype, strides)
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().dla_plan_check(ctypes.byref(d), ctypes.byref(s), ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def plan_check_code(patterns, causal, scale, B, N, H, D=HEAD_DIM, dtype=DLA_BF16, strides=None):
    """Raw return code of dla_plan_check (for error-path tests)."""
    d = make_desc(patterns, causal, scale)
    s = make_shape(B, N, H, D, dtype, strides)
    return lib().dla_plan_check(ctypes.byref(d), ctypes.byref(s), None, None)


def pair_count(patterns, causal, B, N, H, D=HEAD_DIM, dtype=DLA_BF16):
    d = make_desc(patterns, causal, 1.0)
    s = make_shape(B, N, H, D, dtype)
    out = ctypes.c_int64(0)
    _check(lib().dla_pair_count(ctypes.byref(d), ctypes.byref(s), ctypes.byref(out)))
    return out.value


def default_scale(D=HEAD_DIM):
    return 1.0 / math.sqrt(D)


def forward(q, k, v, patterns, causal=True, scale=None, out=None, lse=None, workspace=None,
            stream=None):
    """Dilated attention forward on the GPU; returns (o, lse).

    q, k, v: [B, N, H, 64] float32 or bfloat16 CUDA tensors with one layout.
    lse: [B, H, N] float32.  Buffers not given are allocated with torch.
    """
    import torch
    scale = default_scale(q.shape[-1]) if scale is None else scale
    _same_layout(q, k, v)
    shape = _shape_of(q)
    desc = make_desc(patterns, causal, scale)
    ws_f, _ = ctypes.c_size_t(0), None
    _check(lib().dla_plan_check(ctypes.byref(desc), ctypes.byref(shape), ctypes.byref(ws_f), None))
    B, N, H, _ = q.shape
    o = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if out is None else out
    _same_layout(q, o)
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_lse(lse_t, q)
    if workspace is None:
        workspace = torch.empty(max(ws_f.value, 1), dtype=torch.uint8, device=q.device)
    _check(lib().dla_forward(ctypes.byref(desc), ctypes.byref(shape), q.data_ptr(), k.data_ptr(),
                             v.data_ptr(), o.data_ptr(), lse_t.data_ptr(), workspace.data_ptr(),
                             workspace.numel(), _stream(stream, q.device)))
    return o, lse_t


# Bytes of the library's static scratch that dla_forward_noalloc uses as its workspace.
NOALLOC_SCRATCH_BYTES = 64 << 20


def forward_noalloc(q, k, v, patterns, causal=True, scale=None, out=None, lse=None, stream=None):
    """dla_forward_noalloc: the forward with the library's static scratch as
    its workspace (no workspace argument, nothing allocated by the library).
    The outputs are still the caller's: pass out/lse to allocate nothing at
    all.  Raises DlaError(DLA_E_WORKSPACE) for problems whose workspace
    exceeds NOALLOC_SCRATCH_BYTES.  Calls that overlap on one GPU race."""
    import torch
    scale = default_scale(q.shape[-1]) if scale is None else scale
    _same_layout(q, k, v)
    shape = _shape_of(q)
    desc = make_desc(patterns, causal, scale)
    B, N, H, _ = q.shape
    o = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if out is None else out
    _same_layout(q, o)
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_lse(lse_t, q)
    _check(lib().dla_forward_noalloc(ctypes.byref(desc), ctypes.byref(shape), q.data_ptr(), k.data_ptr(),
                                     v.data_ptr(), o.data_ptr(), lse_t.data_ptr(),
                                     _stream(stream, q.device)))
    return o, lse_t


def backward(q, k, v, o, lse, dout, patterns, causal=True, scale=None, dq=None, dk=None, dv=None,
             workspace=None, stream=None):
    """Gradients (dq, dk, dv) of sum(dout * o) for dla forward outputs (o, lse)."""
    import torch
    scale = default_scale(q.shape[-1]) if scale is None else scale
    _same_layout(q, k, v, o, dout)
    _check_lse(lse, q)
    shape = _shape_of(q)
    desc = make_desc(patterns, causal, scale)
    ws_b = ctypes.c_size_t(0)
    _check(lib().dla_plan_check(ctypes.byref(desc), ctypes.byref(shape), None, ctypes.byref(ws_b)))
    grads = []
    for g in (dq, dk, dv):
        if g is None:
            g = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
        _same_layout(q, g)
        grads.append(g)
    if workspace is None:
        workspace = torch.empty(max(ws_b.value, 1), dtype=torch.uint8, device=q.device)
    _check(lib().dla_backward(ctypes.byref(desc), ctypes.byref(shape), q.data_ptr(), k.data_ptr(),
                              v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                              grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
                              workspace.data_ptr(), workspace.numel(), _stream(stream, q.device)))
    return tuple(grads)


def timing_enable(on: bool = True):
    """Bracket every library kernel launch with HIP events (profiling aid)."""
    _check(lib().dla_timing_enable(int(bool(on))))


def timing_collect(name: str):
    """(launches, total_ms) of the timed launches of kernel family `name`; forgets them."""
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(lib().dla_timing_collect(name.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def row_map(patterns, N, H, pattern, device="cuda", stream=None):
    """Device int32 [H, N/r] map of sparse rows to original rows for one pattern."""
    import torch
    desc = make_desc(patterns, False, 1.0)
    r = patterns[pattern][1]
    out = torch.empty((H, -(-N // r)), dtype=torch.int32, device=device)
    _check(lib().dla_row_map(ctypes.byref(desc), N, H, pattern, out.data_ptr(),
                             _stream(stream, out.device)))
    return out


# ---- sequence shards (one device's share of the sequence-split scheme) ----

def plan_check_shard(patterns, causal, scale, B, N, H, total_rows, shard_start, D=HEAD_DIM,
                     dtype=DLA_BF16, strides=None):
    """(forward, backward) workspace bytes of one shard; raises DlaError on an invalid shard."""
    d = make_desc(patterns, causal, scale)
    s = make_shape(B, N, H, D, dtype, strides)
    sh = Shard(total_rows, shard_start)
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().dla_plan_check_shard(ctypes.byref(d), ctypes.byref(s), ctypes.byref(sh), ctypes.byref(f),
                                      ctypes.byref(b)))
    return f.value, b.value


def plan_check_shard_code(patterns, causal, scale, B, N, H, total_rows, shard_start, D=HEAD_DIM,
                          dtype=DLA_BF16):
    """Raw return code of dla_plan_check_shard (for error-path tests)."""
    d = make_desc(patterns, causal, scale)
    s = make_shape(B, N, H, D, dtype)
    sh = Shard(total_rows, shard_start)
    return lib().dla_plan_check_shard(ctypes.byref(d), ctypes.byref(s), ctypes.byref(sh), None, None)


def pair_count_shard(patterns, causal, B, N, H, total_rows, shard_start):
    d = make_desc(patterns, causal, 1.0)
    s = make_shape(B, N, H, HEAD_DIM, DLA_BF16)
    sh = Shard(total_rows, shard_start)
    out = ctypes.c_int64(0)
    _check(lib().dla_pair_count_shard(ctypes.byref(d), ctypes.byref(s), ctypes.byref(sh), ctypes.byref(out)))
    return out.value


def shard_gather(x, patterns, pattern, total_rows, shard_start, causal=True, out=None, stream=None):
    """This shard's part of the exchange of spanning pattern `pattern`: [B, H, N/r, D]."""
    import torch
    shape = _shape_of(x)
    desc = make_desc(patterns, causal, 1.0)
    sh = Shard(total_rows, shard_start)
    B, N, H, D = x.shape
    r = patterns[pattern][1]
    if out is None:
        out = torch.empty((B, H, N // r, D), dtype=x.dtype, device=x.device)
    if out.shape != (B, H, N // r, D) or not out.is_contiguous() or out.dtype != x.dtype:
        raise DlaError(DLA_E_INVALID, "out must be a contiguous [B, H, N/r, D] tensor of x's dtype")
    _check(lib().dla_shard_gather(ctypes.byref(desc), ctypes.byref(shape), ctypes.byref(sh), pattern,
                                  x.data_ptr(), out.data_ptr(), _stream(stream, x.device)))
    return out


def forward_shard(q, k, v, patterns, total_rows, shard_start, ext_k=None, ext_v=None, causal=True,
                  scale=None, out=None, lse=None, workspace=None, stream=None):
    """Forward pass of one shard; returns (o, lse) for the shard's rows.

    ext_k / ext_v: dicts {pattern index: [w/N, B, H, N/r, D] gathered tensor}
    for the patterns whose segments span shards.
    """
    import torch
    scale = default_scale(q.shape[-1]) if scale is None else scale
    _same_layout(q, k, v)
    shape = _shape_of(q)
    desc = make_desc(patterns, causal, scale)
    sh = Shard(total_rows, shard_start)
    ws_f = ctypes.c_size_t(0)
    _check(lib().dla_plan_check_shard(ctypes.byref(desc), ctypes.byref(shape), ctypes.byref(sh),
                                      ctypes.byref(ws_f), None))
    B, N, H, _ = q.shape
    o = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if out is None else out
    _same_layout(q, o)
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_lse(lse_t, q)
    P = len(patterns)
    ek = (ctypes.c_void_p * P)()
    ev = (ctypes.c_void_p * P)()
    for i, (w, r) in enumerate(patterns):
        if w > N:
            tk, tv = (ext_k or {}).get(i), (ext_v or {}).get(i)
            want = (w // N, B, H, N // r, q.shape[-1])
            for t in (tk, tv):
                if t is None or tuple(t.shape) != want or not t.is_contiguous() or t.dtype != q.dtype:
                    raise DlaError(DLA_E_INVALID, f"pattern {i} spans shards: needs contiguous "
                                   f"gathered k and v of shape {want}")
            ek[i], ev[i] = tk.data_ptr(), tv.data_ptr()
    if workspace is None:
        workspace = torch.empty(max(ws_f.value, 1), dtype=torch.uint8, device=q.device)
    _check(lib().dla_forward_shard(ctypes.byref(desc), ctypes.byref(shape), ctypes.byref(sh),
                                   q.data_ptr(), k.data_ptr(), v.data_ptr(), ek, ev, o.data_ptr(),
                                   lse_t.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                   _stream(stream, q.device)))
    return o, lse_t


def _ptr_array(P, tensors):
    arr = (ctypes.c_void_p * P)()
    for i, t in (tensors or {}).items():
        arr[i] = t.data_ptr()
    return arr


def backward_shard(q, k, v, o, lse, dout, patterns, total_rows, shard_start, ext_k=None, ext_v=None,
                   causal=True, scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """First half of one shard's backward.

    Returns (dq, dk, dv, ext_dk, ext_dv, workspace): dq final; dk/dv final on
    rows no spanning pattern keeps; ext_dk/ext_dv dicts {pattern: fp32
    [w/N, B, H, N/r, D]} of this shard's contributions, to be summed over the
    segment's devices and handed to finish_shard with the same workspace.
    """
    import torch
    scale = default_scale(q.shape[-1]) if scale is None else scale
    _same_layout(q, k, v, o, dout)
    _check_lse(lse, q)
    shape = _shape_of(q)
    desc = make_desc(patterns, causal, scale)
    sh = Shard(total_rows, shard_start)
    ws_b = ctypes.c_size_t(0)
    _check(lib().dla_plan_check_shard(ctypes.byref(desc), ctypes.byref(shape), ctypes.byref(sh), None,
                                      ctypes.byref(ws_b)))
    B, N, H, D = q.shape
    grads = []
    for g in (dq, dk, dv):
        if g is None:
            g = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
        _same_layout(q, g)
        grads.append(g)
    P = len(patterns)
    out_k, out_v = {}, {}
    for i, (w, r) in enumerate(patterns):
        if w > N:
            out_k[i] = torch.empty((w // N, B, H, N // r, D), dtype=torch.float32, device=q.device)
            out_v[i] = torch.empty_like(out_k[i])
    if workspace is None:
        workspace = torch.empty(max(ws_b.value, 1), dtype=torch.uint8, device=q.device)
    _check(lib().dla_backward_shard(ctypes.byref(desc), ctypes.byref(shape), ctypes.byref(sh),
                                    q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    dout.data_ptr(), _ptr_array(P, ext_k), _ptr_array(P, ext_v),
                                    grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
                                    _ptr_array(P, out_k), _ptr_array(P, out_v), workspace.data_ptr(),
                                    workspace.numel(), _stream(stream, q.device)))
    return grads[0], grads[1], grads[2], out_k, out_v, workspace


def finish_shard(dk, dv, patterns, total_rows, shard_start, red_dk, red_dv, workspace, causal=True,
                 scale=None, stream=None):
    """Second half: dk/dv of the rows spanning patterns keep, from the exchanged parts
    red_dk/red_dv ({pattern: fp32 [B, H, N/r, D]}) and the workspace of backward_shard."""
    scale = default_scale(dk.shape[-1]) if scale is None else scale
    _same_layout(dk, dv)
    shape = _shape_of(dk)
    desc = make_desc(patterns, causal, scale)
    sh = Shard(total_rows, shard_start)
    P = len(patterns)
    _check(lib().dla_shard_finish(ctypes.byref(desc), ctypes.byref(shape), ctypes.byref(sh),
                                  _ptr_array(P, red_dk), _ptr_array(P, red_dv), dk.data_ptr(),
                                  dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                  _stream(stream, dk.device)))
    return dk, dv


# ---- batches of different lengths ----

def _lengths_tensor(lengths, B, device):
    import torch
    t = torch.as_tensor(lengths, dtype=torch.int32)
    if t.shape != (B,):
        raise DlaError(DLA_E_INVALID, f"lengths must have B = {B} entries")
    return t.to(device).contiguous()


def forward_varlen(q, k, v, lengths, patterns, causal=True, scale=None, out=None, lse=None,
                   workspace=None, stream=None):
    """Forward on a padded batch: batch b is its first lengths[b] rows; returns (o, lse)."""
    import torch
    scale = default_scale(q.shape[-1]) if scale is None else scale
    _same_layout(q, k, v)
    shape = _shape_of(q)
    desc = make_desc(patterns, causal, scale)
    ws_f = ctypes.c_size_t(0)
    _check(lib().dla_plan_check(ctypes.byref(desc), ctypes.byref(shape), ctypes.byref(ws_f), None))
    B, N, H, _ = q.shape
    lt = _lengths_tensor(lengths, B, q.device)
    o = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if out is None else out
    _same_layout(q, o)
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_lse(lse_t, q)
    if workspace is None:
        workspace = torch.empty(max(ws_f.value, 1), dtype=torch.uint8, device=q.device)
    _check(lib().dla_forward_varlen(ctypes.byref(desc), ctypes.byref(shape), lt.data_ptr(), q.data_ptr(),
                                    k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_t.data_ptr(),
                                    workspace.data_ptr(), workspace.numel(), _stream(stream, q.device)))
    return o, lse_t


def backward_varlen(q, k, v, o, lse, dout, lengths, patterns, causal=True, scale=None, dq=None,
                    dk=None, dv=None, workspace=None, stream=None):
    """Gradients on a padded batch (padding rows get zero gradients)."""
    import torch
    scale = default_scale(q.shape[-1]) if scale is None else scale
    _same_layout(q, k, v, o, dout)
    _check_lse(lse, q)
    shape = _shape_of(q)
    desc = make_desc(patterns, causal, scale)
    ws_b = ctypes.c_size_t(0)
    _check(lib().dla_plan_check(ctypes.byref(desc), ctypes.byref(shape), None, ctypes.byref(ws_b)))
    lt = _lengths_tensor(lengths, q.shape[0], q.device)
    grads = []
    for g in (dq, dk, dv):
        if g is None:
            g = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
        _same_layout(q, g)
        grads.append(g)
    if workspace is None:
        workspace = torch.empty(max(ws_b.value, 1), dtype=torch.uint8, device=q.device)
    _check(lib().dla_backward_varlen(ctypes.byref(desc), ctypes.byref(shape), lt.data_ptr(), q.data_ptr(),
                                     k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     dout.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(),
                                     grads[2].data_ptr(), workspace.data_ptr(), workspace.numel(),
                                     _stream(stream, q.device)))
    return tuple(grads)


def pair_count_varlen(patterns, causal, lengths, N, H):
    d = make_desc(patterns, causal, 1.0)
    s = make_shape(len(lengths), N, H, HEAD_DIM, DLA_BF16)
    arr = (ctypes.c_int32 * max(1, len(lengths)))(*[int(x) for x in lengths])
    out = ctypes.c_int64(0)
    _check(lib().dla_pair_count_varlen(ctypes.byref(d), ctypes.byref(s), arr, ctypes.byref(out)))
    return out.value


# ---- a LongNet attention layer (projections by hipBLASLt, attention by the library) ----

class Blas:
    """The hipBLASLt handle the layer calls use."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib().dla_blas_create(ctypes.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            lib().dla_blas_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def layer_plan_check(patterns, causal, scale, B, N, H):
    d = make_desc(patterns, causal, scale)
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().dla_layer_plan_check(ctypes.byref(d), B, N, H, ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def layer_forward(x, w_qkv, w_o, patterns, blas, causal=True, scale=None, workspace=None, stream=None):
    """Y = DA(X W_q, X W_k, X W_v) W_o; returns (y, qkv, attn, lse) (the last three for the backward)."""
    import torch
    B, N, E = x.shape
    H = E // HEAD_DIM
    scale = default_scale() if scale is None else scale
    for t, shp in ((x, (B, N, E)), (w_qkv, (E, 3 * E)), (w_o, (E, E))):
        if tuple(t.shape) != shp or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise DlaError(DLA_E_INVALID, f"expected a contiguous bfloat16 tensor of shape {shp}")
    desc = make_desc(patterns, causal, scale)
    ws_f, _ = layer_plan_check(patterns, causal, scale, B, N, H)
    qkv = torch.empty((3, B, N, H, HEAD_DIM), dtype=torch.bfloat16, device=x.device)
    attn = torch.empty((B, N, H, HEAD_DIM), dtype=torch.bfloat16, device=x.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=x.device)
    y = torch.empty((B, N, E), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(ws_f, dtype=torch.uint8, device=x.device)
    _check(lib().dla_layer_forward(ctypes.byref(desc), B, N, H, x.data_ptr(), w_qkv.data_ptr(),
                                   w_o.data_ptr(), qkv.data_ptr(), attn.data_ptr(), lse.data_ptr(),
                                   y.data_ptr(), blas.handle, workspace.data_ptr(), workspace.numel(),
                                   _stream(stream, x.device)))
    return y, qkv, attn, lse


def layer_backward(x, w_qkv, w_o, qkv, attn, lse, dy, patterns, blas, causal=True, scale=None,
                   workspace=None, stream=None):
    """(dx, dw_qkv, dw_o) of sum(dy * y); weight gradients in float32."""
    import torch
    B, N, E = x.shape
    H = E // HEAD_DIM
    scale = default_scale() if scale is None else scale
    desc = make_desc(patterns, causal, scale)
    _, ws_b = layer_plan_check(patterns, causal, scale, B, N, H)
    dx = torch.empty_like(x)
    dw_qkv = torch.empty((E, 3 * E), dtype=torch.float32, device=x.device)
    dw_o = torch.empty((E, E), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(ws_b, dtype=torch.uint8, device=x.device)
    _check(lib().dla_layer_backward(ctypes.byref(desc), B, N, H, x.data_ptr(), w_qkv.data_ptr(),
                                    w_o.data_ptr(), qkv.data_ptr(), attn.data_ptr(), lse.data_ptr(),
                                    dy.contiguous().data_ptr(), dx.data_ptr(), dw_qkv.data_ptr(),
                                    dw_o.data_ptr(), blas.handle, workspace.data_ptr(),
                                    workspace.numel(), _stream(stream, x.device)))
    return dx, dw_qkv, dw_o


# ---- 8-bit keys and values ----

def quantize_fp8(x, stream=None):
    """FP8 E4M3 codes of a bf16 [B, N, H, 64] tensor and its per-(batch, head)
    fp32 scales: returns (codes uint8 with x's layout, scale [B, H])."""
    import torch
    if x.dtype != torch.bfloat16:
        raise DlaError(DLA_E_UNSUPPORTED, "quantization reads bfloat16")
    shape = _shape_of(x)
    B, N, H, _ = x.shape
    x8 = torch.empty_strided(x.shape, x.stride(), dtype=torch.uint8, device=x.device)
    scale = torch.empty((B, H), dtype=torch.float32, device=x.device)
    _check(lib().dla_quantize_fp8(ctypes.byref(shape), x.data_ptr(), x8.data_ptr(), scale.data_ptr(),
                                  _stream(stream, x.device)))
    return x8, scale


def forward_fp8kv(q, k8, v8, k_scale, v_scale, patterns, causal=True, scale=None, out=None, lse=None,
                  workspace=None, stream=None):
    """dla forward with FP8 E4M3 keys and values (codes with q's layout, [B, H] scales)."""
    import torch
    scale = default_scale(q.shape[-1]) if scale is None else scale
    for t in (k8, v8):
        if t.shape != q.shape or t.stride() != q.stride() or t.dtype != torch.uint8 or t.device != q.device:
            raise DlaError(DLA_E_INVALID, "k8 and v8 must be uint8 tensors with q's shape and strides")
    B, N, H, _ = q.shape
    for t in (k_scale, v_scale):
        if tuple(t.shape) != (B, H) or not t.is_contiguous() or t.dtype != torch.float32:
            raise DlaError(DLA_E_INVALID, "scales must be contiguous float32 [B, H] tensors")
    shape = _shape_of(q)
    desc = make_desc(patterns, causal, scale)
    ws_f = ctypes.c_size_t(0)
    _check(lib().dla_plan_check(ctypes.byref(desc), ctypes.byref(shape), ctypes.byref(ws_f), None))
    o = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if out is None else out
    _same_layout(q, o)
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_lse(lse_t, q)
    if workspace is None:
        workspace = torch.empty(max(ws_f.value, 1), dtype=torch.uint8, device=q.device)
    _check(lib().dla_forward_fp8kv(ctypes.byref(desc), ctypes.byref(shape), q.data_ptr(), k8.data_ptr(),
                                   v8.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(), o.data_ptr(),
                                   lse_t.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                   _stream(stream, q.device)))
    return o, lse_t
