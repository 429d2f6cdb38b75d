"""Plain CPU oracle for a LongNet attention layer.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import or call this module.

[G] 实验设计 (the gptget.net summary of arXiv 2307.02486, experiment design)
gives the model the method was trained in: 768 model dimensions and 12 heads.
The pages say nothing more about the layer, so it is read as the plain
multi-head attention block with dilated attention in place of dense
attention: Q = X W_q, K = X W_k, V = X W_v (split into H heads of E / H
columns each), A = DA(Q, K, V), Y = A W_o, with W_qkv = [W_q | W_k | W_v] and
no bias, normalisation or residual.  X, Y are [B, N, E]; W_qkv is [E, 3E] and
W_o is [E, E], both applied as y = x W.  Arithmetic is float64; the matrix
products are numpy's, the attention is `dilated.forward` / `dilated.backward`.
"""
from __future__ import annotations

import numpy as np

from .dilated import backward, forward, forward_rows


def _split(qkv, H):
    B, N, E3 = qkv.shape
    E = E3 // 3
    return [qkv[..., j * E:(j + 1) * E].reshape(B, N, H, E // H) for j in range(3)]


def layer_forward(x, w_qkv, w_o, H, patterns, causal, scale, workers=1, attn_dtype=np.float64):
    """Y [B, N, E] and the saved activations (q, k, v, attn, lse) of the layer.
    `attn_dtype` is the precision of the attention step (the projections
    stay float64); float32 serves large checks of bf16 results."""
    x, w_qkv, w_o = (np.asarray(t, np.float64) for t in (x, w_qkv, w_o))
    B, N, E = x.shape
    q, k, v = _split(x @ w_qkv, H)
    attn, lse = forward(q, k, v, patterns, causal, scale, dtype=attn_dtype, workers=workers)
    attn, lse = np.asarray(attn, np.float64), np.asarray(lse, np.float64)
    y = attn.reshape(B, N, E) @ w_o
    return y, (q, k, v, attn, lse)


def layer_backward(x, w_qkv, w_o, saved, dy, patterns, causal, scale, workers=1, attn_dtype=np.float64):
    """(dX, dW_qkv, dW_o) of sum(dY * Y) by the chain rule through the layer.

    Y = A W_o gives dA = dY W_o^T and dW_o = A^T dY (summed over batch and
    rows); the attention backward maps dA to dQ, dK, dV; the projections give
    dX = [dQ | dK | dV] W_qkv^T and dW_qkv = X^T [dQ | dK | dV].
    """
    x, w_qkv, w_o, dy = (np.asarray(t, np.float64) for t in (x, w_qkv, w_o, dy))
    q, k, v, attn, lse = saved
    B, N, E = x.shape
    a2 = attn.reshape(B * N, E)
    dy2 = dy.reshape(B * N, E)
    dw_o = a2.T @ dy2
    da = (dy2 @ w_o.T).reshape(attn.shape)
    dq, dk, dv = backward(q, k, v, attn, lse, da, patterns, causal, scale, dtype=attn_dtype,
                          workers=workers)
    dq, dk, dv = (np.asarray(t, np.float64) for t in (dq, dk, dv))
    dp = np.concatenate([t.reshape(B * N, E) for t in (dq, dk, dv)], axis=1)
    dx = (dp @ w_qkv.T).reshape(B, N, E)
    dw_qkv = x.reshape(B * N, E).T @ dp
    return dx, dw_qkv, dw_o


def layer_forward_rows(x, w_qkv, w_o, H, patterns, causal, scale, b, rows):
    """Rows `rows` of batch b of Y, one query row at a time (for spot checks)."""
    x, w_qkv, w_o = (np.asarray(t, np.float64) for t in (x, w_qkv, w_o))
    E = x.shape[2]
    q, k, v = _split(x[b:b + 1] @ w_qkv, H)
    attn = np.stack([forward_rows(q, k, v, patterns, causal, scale, 0, h, rows)[0]
                     for h in range(H)], axis=1)  # [rows, H, D]
    return attn.reshape(len(rows), E) @ w_o
