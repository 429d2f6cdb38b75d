"""Seeded synthetic inputs and the workload shapes, shared by tests, bench and smoke.

This module holds no arithmetic of the attention method itself: it only draws
random tensors, rounds them to bfloat16 bit patterns and describes the
workloads.  Both the CPU oracle's callers and the GPU path's callers take
their inputs from here, so the two sides always see identical values.

Workloads (the model settings quoted by the gptget.net summary of arXiv
2307.02486, section 实验设计 (experiment design): 768-dim model, 12 heads, so
head_dim 64; sequences 2K..32K, extended here to the 1M-token one-GPU share).
The segment lengths w and dilation rates r follow the geometric schedule
w = 2048 * 2**i, r = 2**i of the same page, section 方法论 (method).
The Stack dataset that page trains on is not available; iid N(0, 1) inputs of
the same shapes stand in for it.
"""
from __future__ import annotations

import dataclasses

import numpy as np

HEAD_DIM = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16"
    B: int
    N: int
    H: int
    patterns: tuple            # ((w, r), ...)
    causal: bool
    backward: bool             # forward+backward workload
    seed: int
    D: int = HEAD_DIM

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def describe(self) -> str:
        pats = ",".join(f"({w},{r})" for w, r in self.patterns)
        return (f"{self.name}: {'fwd+bwd' if self.backward else 'fwd'} {self.dtype} B={self.B} "
                f"N={self.N} H={self.H} D={self.D} {'causal' if self.causal else 'non-causal'} "
                f"patterns {pats}")


def geometric_patterns(w0: int, alpha: int, count: int) -> tuple:
    return tuple((w0 * alpha ** i, alpha ** i) for i in range(count))


WORKLOADS = {
    "C1": Workload("C1", "f32", 1, 2048, 12, ((512, 1), (1024, 2), (2048, 4)), False, False, 1),
    "C2": Workload("C2", "bf16", 4, 8192, 12, ((2048, 1), (4096, 2), (8192, 4)), True, False, 2),
    "C3": Workload("C3", "bf16", 1, 32768, 12, geometric_patterns(2048, 2, 5), True, False, 3),
    "C4": Workload("C4", "bf16", 1, 1 << 20, 12, geometric_patterns(2048, 2, 10), True, False, 4),
    "C5": Workload("C5", "bf16", 2, 32768, 12, geometric_patterns(2048, 2, 5), True, True, 5),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array holding exactly the bfloat16-representable values of x."""
    return bf16_bits_to_f32(bf16_bits(x))


def draw(shape, seed: int, count: int, dtype: str = "f32", chunk_rows: int = 1 << 16):
    """Draw `count` tensors of `shape` from numpy's PCG64(seed), in order.

    Each tensor is standard_normal(shape, float32), drawn in slices along the
    first two axes so that huge shapes do not need a float64 temporary.  For
    dtype "bf16" the values are rounded to bfloat16 (ties to even) and returned
    as float32 arrays that hold those exact values.
    """
    gen = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(count):
        t = np.empty(shape, dtype=np.float32)
        flat = t.reshape(-1, *shape[2:]) if len(shape) > 2 else t.reshape(-1)
        for i in range(0, flat.shape[0], chunk_rows):
            blk = flat[i:i + chunk_rows]
            blk[...] = gen.standard_normal(blk.shape, dtype=np.float32)
            if dtype == "bf16":
                blk[...] = round_to_bf16(blk)
        out.append(t)
    return out


def workload_inputs(wl: Workload, B: int | None = None, N: int | None = None):
    """(q, k, v[, dout]) for a workload, as float32 arrays [B, N, H, D]."""
    shape = (wl.B if B is None else B, wl.N if N is None else N, wl.H, wl.D)
    return draw(shape, wl.seed, 4 if wl.backward else 3, wl.dtype)


def random_case(seed: int, B: int, N: int, H: int, dtype: str = "f32", count: int = 3, D: int = HEAD_DIM):
    """Small seeded case for property and parity tests."""
    return draw((B, N, H, D), seed, count, dtype)


def layer_inputs(seed: int, B: int, N: int, H: int, dtype: str = "bf16", D: int = HEAD_DIM):
    """(x, w_qkv, w_o, dy) for an attention layer of E = H * D model dimensions.

    x and dy are [B, N, E] standard normal; w_qkv [E, 3E] and w_o [E, E] are
    standard normal scaled by 1 / sqrt(E) (so that projections of unit-variance
    rows keep unit variance), all drawn from numpy's PCG64(seed) in that order
    and, for dtype "bf16", rounded to bfloat16 after scaling.
    """
    E = H * D
    gen = np.random.Generator(np.random.PCG64(seed))
    x = gen.standard_normal((B, N, E), dtype=np.float32)
    w_qkv = gen.standard_normal((E, 3 * E), dtype=np.float32) * np.float32(1.0 / np.sqrt(E))
    w_o = gen.standard_normal((E, E), dtype=np.float32) * np.float32(1.0 / np.sqrt(E))
    dy = gen.standard_normal((B, N, E), dtype=np.float32)
    out = [x, w_qkv, w_o, dy]
    if dtype == "bf16":
        out = [round_to_bf16(t) for t in out]
    return out
