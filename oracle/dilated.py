"""Plain CPU oracle for LongNet dilated attention.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import or call this module.  The product path (the HIP library and its
Python binding) never does, and shares no code with it.

Sources (web pages about LongNet, arXiv 2307.02486):
  [G] the gptget.net summary page of arXiv 2307.02486, sections 方法论 (method),
      方法详解 (method details), 实验设计 (experiment design), 术语表 (glossary)
      and 原文摘要 (the English abstract);
  [D] the darcstar.tech research page "LongNet: Scaling Transformers to
      1,000,000,000 Tokens", its abstract and the DarcStar commentary.

What the method computes.  The pages describe it in words only (they print no
equations, worked examples or code):
  * the sequence is split into equal-length segments of length w
    ([G] 方法论 and 方法详解, first item);
  * each segment is sampled at a dilation rate r, i.e. every r-th row is kept,
    for the queries, keys and values alike ([G] 方法论 / 方法详解, second and
    fourth items);
  * each head uses a different offset; head h starts at row h mod r
    ([G] 方法论 / 方法详解, third item);
  * dense softmax attention runs inside each sparsified segment;
  * several (w, r) patterns are mixed ([G] 方法详解, seventh item; 术语表
    "多尺度"), each pattern's output weighted by its softmax denominator so
    that the normaliser the patterns share stays exact ([D] commentary, the
    paragraph on combining the softmax over scattered pieces).

Readings where the pages are silent (each is also listed with the design
notes): causal masking applies inside each sparsified segment by original
position; a row no pattern selects gets output 0 and log-sum-exp -inf; the
pattern weight is exp(LSE_p - LSE) with the unshifted denominators; duplicate
patterns count with multiplicity; w % r == 0 is required; when N is not a
multiple of w (or w > N) the last segment holds the remaining rows only, so
a sequence behaves as if padded to a multiple of w with rows that never
take part (the padded rows would otherwise be keys of real queries).
Batches of different lengths (`lengths`): batch b is the sequence of its
first lengths[b] rows; the rows after it are padding and get output 0,
log-sum-exp -inf and zero gradients.

Layouts: q, k, v, o, dout, dq, dk, dv are [B, N, H, D]; lse is [B, H, N] in
natural log.  Arithmetic is float64 unless `dtype` asks for float32 (the timed
CPU baseline); a library matmul and numpy's exp/log are the only primitives.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np


def check_patterns(N: int, patterns) -> None:
    for w, r in patterns:
        if not (w > 0 and r > 0 and w % r == 0):
            raise ValueError(f"pattern (w={w}, r={r}) needs w % r == 0")


def segments(N: int, w: int) -> int:
    """Number of segments: the last one holds the N mod w remaining rows, if any."""
    return -(-N // w)


def segment_rows(N: int, w: int, r: int, h: int, s: int) -> np.ndarray:
    """Original rows of segment s of pattern (w, r) for head h, in sparse order:
    s*w + (h mod r) + a*r for every a whose row lies inside the segment and the
    sequence ([G] 方法论: segments of length w, every r-th row, head offset
    h mod r; a last segment shorter than w keeps the rows it has)."""
    idx = s * w + (h % r) + r * np.arange(w // r, dtype=np.int64)
    return idx[idx < N]


def row_map(N: int, w: int, r: int, h: int) -> np.ndarray:
    """Original row of every sparse row of pattern (w, r) for head h.

    Entry s*(w/r) + a is row a of segment s after dilation: s*w + (h mod r) + a*r
    ([G] 方法论: segments of length w, every r-th row, head offset h mod r),
    for the first ceil(N/r) entries; an entry whose row lies past the end of
    the sequence (in a shorter last segment) is -1.
    """
    L = w // r
    seg = np.arange(segments(N, w), dtype=np.int64)[:, None]
    a = np.arange(L, dtype=np.int64)[None, :]
    rows = (seg * w + (h % r) + a * r).reshape(-1)[: -(-N // r)]
    return np.where(rows < N, rows, -1)


def segment_attention(qs, ks, vs, scale, causal):
    """Dense softmax attention of one sparsified segment; returns (O, LSE).

    qs, ks, vs are [L, D].  With `causal`, sparse row a attends to sparse rows
    a' <= a only, which is original position k <= q inside the segment.
    """
    S = scale * (qs @ ks.T)
    if causal:
        S = np.where(np.tri(S.shape[0], dtype=bool), S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    den = E.sum(axis=1, keepdims=True)
    return (E / den) @ vs, (m + np.log(den))[:, 0]


def combine(o_parts, lse_parts):
    """Merge per-pattern results with weights exp(LSE_p - LSE) ([D] commentary).

    o_parts: list of [..., D] arrays, lse_parts: list of [...] arrays (same
    leading layout as o_parts) holding -inf where a pattern does not select
    the row.  LSE = log sum_p exp(LSE_p);
    rows no pattern selects get O = 0 and LSE = -inf, computed with explicit
    masking so that no (-inf) - (-inf) is ever formed.
    """
    lse_stack = np.stack(lse_parts)
    m = lse_stack.max(axis=0)
    covered = np.isfinite(m)
    m0 = np.where(covered, m, 0.0)
    total = np.exp(lse_stack - m0).sum(axis=0)
    lse = np.where(covered, m0 + np.log(np.where(covered, total, 1.0)), -np.inf)
    weight = np.where(covered, np.exp(lse_stack - np.where(covered, lse, 0.0)), 0.0)
    o = np.einsum("p...,p...d->...d", weight, np.stack(o_parts))
    return o.astype(lse_stack.dtype), lse.astype(lse_stack.dtype)


def _units(patterns, B, H, N):
    return [(p, b, h, s) for p, (w, r) in enumerate(patterns)
            for b in range(B) for h in range(H) for s in range(segments(N, w))]


def _run(units, fn, workers):
    if workers <= 1:
        for u in units:
            fn(u)
        return
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        for _ in ex.map(fn, units):
            pass


def _lengths(lengths, B, N):
    return [N] * B if lengths is None else [int(x) for x in lengths]


def forward(q, k, v, patterns, causal, scale, dtype=np.float64, workers=1, lengths=None,
            heads=None):
    """Dilated attention forward; returns (O [B,N,H,D], LSE [B,H,N]).

    An explicit loop over pattern, batch, head and segment: gather the rows the
    pattern keeps, attend densely inside the segment, scatter the result back
    into a per-pattern buffer (rows a pattern does not select keep O_p = 0,
    LSE_p = -inf), then merge the patterns with `combine`.  With `lengths`,
    batch b's sequence is its first lengths[b] rows.  `heads` names the head
    index of each entry of the inputs' head axis (default 0..H-1), so that a
    slice q[:, :, h:h+1] with heads=[h] gives head h's result alone (the head
    index sets the row offset h mod r).
    """
    q, k, v = (np.asarray(t, dtype=dtype) for t in (q, k, v))
    B, N, H, D = q.shape
    check_patterns(N, patterns)
    lens = _lengths(lengths, B, N)
    head_ids = list(range(H)) if heads is None else [int(x) for x in heads]
    if len(head_ids) != H:
        raise ValueError(f"heads names {len(head_ids)} heads for an input with {H}")
    o_parts = [np.zeros((B, N, H, D), dtype) for _ in patterns]
    lse_parts = [np.full((B, H, N), -np.inf, dtype) for _ in patterns]

    def unit(u):
        p, b, j, s = u          # j: position on the inputs' head axis
        w, r = patterns[p]
        idx = segment_rows(lens[b], w, r, head_ids[j], s)
        if idx.size == 0:
            return
        o, lse = segment_attention(q[b, idx, j], k[b, idx, j], v[b, idx, j], scale, causal)
        o_parts[p][b, idx, j] = o
        lse_parts[p][b, j, idx] = lse

    _run(_units(patterns, B, H, N), unit, workers)
    o, lse = combine(o_parts, [x.transpose(0, 2, 1) for x in lse_parts])
    return o, np.ascontiguousarray(lse.transpose(0, 2, 1))


def forward_rows(q, k, v, patterns, causal, scale, b, h, rows, dtype=np.float64):
    """Forward output of selected rows only: (O [len(rows), D], LSE [len(rows)]).

    The same definition evaluated one query row at a time, for spot checks at
    sizes where the full oracle is too slow: for every pattern that selects
    row n for head h, attend from n to the rows of its sparsified segment.
    """
    out_o, out_lse = [], []
    for n in rows:
        n = int(n)
        o_parts, lse_parts = [], []
        for w, r in patterns:
            if n % r != h % r:
                continue
            idx = segment_rows(q.shape[1], w, r, h, n // w)
            if causal:
                idx = idx[idx <= n]
            scores = scale * (np.asarray(k[b, idx, h], dtype) @ np.asarray(q[b, n, h], dtype))
            m = scores.max()
            e = np.exp(scores - m)
            o_parts.append((e @ np.asarray(v[b, idx, h], dtype)) / e.sum())
            lse_parts.append(m + np.log(e.sum()))
        if not lse_parts:
            out_o.append(np.zeros(q.shape[-1], dtype))
            out_lse.append(-np.inf)
            continue
        o, lse = combine([x[None] for x in o_parts], [np.array([x], dtype) for x in lse_parts])
        out_o.append(o[0])
        out_lse.append(lse[0])
    return np.array(out_o, dtype), np.array(out_lse, dtype)


def backward_dq_rows(q, k, v, dout, patterns, causal, scale, b, h, rows, dtype=np.float64):
    """dQ of selected rows only ([len(rows), D]), for spot checks at sizes where
    the full backward is too slow.

    Row n's gradient needs only its own keys: for every pattern that keeps n
    (head h), the rows of its dilated segment (at or before n if causal).
    With the combined LSE and O of the row (as in `forward_rows`) and
    D = dO_n . O_n, dQ_n = scale * sum over those (pattern, key) pairs of
    P (dP - D) K_key, where P = exp(S - LSE) and dP = dO_n . V_key.
    """
    out = []
    for n in rows:
        n = int(n)
        parts = []
        for w, r in patterns:
            if n % r != h % r:
                continue
            idx = segment_rows(q.shape[1], w, r, h, n // w)
            if causal:
                idx = idx[idx <= n]
            parts.append(idx)
        if not parts:
            out.append(np.zeros(q.shape[-1], dtype))
            continue
        qn = np.asarray(q[b, n, h], dtype)
        don = np.asarray(dout[b, n, h], dtype)
        S = [scale * (np.asarray(k[b, idx, h], dtype) @ qn) for idx in parts]
        m = max(s.max() for s in S)
        den = sum(np.exp(s - m).sum() for s in S)
        lse = m + np.log(den)
        o = sum(np.exp(s - lse) @ np.asarray(v[b, idx, h], dtype) for s, idx in zip(S, parts))
        d = don @ o
        dq = np.zeros(q.shape[-1], dtype)
        for s, idx in zip(S, parts):
            P = np.exp(s - lse)
            dP = np.asarray(v[b, idx, h], dtype) @ don
            dq += scale * ((P * (dP - d)) @ np.asarray(k[b, idx, h], dtype))
        out.append(dq)
    return np.array(out, dtype)


def backward(q, k, v, o, lse, dout, patterns, causal, scale, dtype=np.float64, workers=1,
             lengths=None):
    """Analytic gradients (dQ, dK, dV) of the combined forward w.r.t. q, k, v.

    The combined output is one softmax over the union (with multiplicity) of
    each row's (pattern, key) pairs, so the usual attention gradient applies
    with the combined LSE and D = rowsum(dO * O): per pattern and segment
    P = exp(S - LSE), dV += P^T dO, dP = dO V^T, dS = P * (dP - D),
    dQ += scale dS K, dK += scale dS^T Q.  Patterns run one after another;
    inside a pattern every (batch, head, segment) writes disjoint rows.
    """
    q, k, v, o, dout = (np.asarray(t, dtype=dtype) for t in (q, k, v, o, dout))
    lse = np.asarray(lse, dtype=dtype)
    B, N, H, D = q.shape
    check_patterns(N, patterns)
    lens = _lengths(lengths, B, N)
    delta = np.einsum("bnhd,bnhd->bhn", dout, o)
    dq, dk, dv = (np.zeros((B, N, H, D), dtype) for _ in range(3))
    for p, (w, r) in enumerate(patterns):

        def unit(u, w=w, r=r):
            _, b, h, s = u
            idx = segment_rows(lens[b], w, r, h, s)
            L = idx.size
            if L == 0:
                return
            qs, ks, vs, dos = q[b, idx, h], k[b, idx, h], v[b, idx, h], dout[b, idx, h]
            S = scale * (qs @ ks.T)
            if causal:
                S = np.where(np.tri(L, dtype=bool), S, -np.inf)
            P = np.exp(S - lse[b, h, idx][:, None])
            dv[b, idx, h] += P.T @ dos
            dP = dos @ vs.T
            dS = P * (dP - delta[b, h, idx][:, None])
            dq[b, idx, h] += scale * (dS @ ks)
            dk[b, idx, h] += scale * (dS.T @ qs)

        units = [(p, b, h, s) for b in range(B) for h in range(H) for s in range(segments(N, w))]
        _run(units, unit, workers)
    return dq, dk, dv


def brute_force_forward(q, k, v, patterns, causal, scale, lengths=None):
    """Union-softmax form on a dense N x N matrix; for tiny inputs only.

    M_h[q, k] counts the patterns whose dilated segment holds both q and k:
    [q = h mod r][k = h mod r][q // w == k // w] (times [k <= q] if causal).
    Then O = (M * e^S) V / rowsum(M * e^S) and LSE = log rowsum(M * e^S).
    This shares no structure with `forward` and pins its combine step.
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, N, H, D = q.shape
    lens = _lengths(lengths, B, N)
    o = np.zeros((B, N, H, D))
    lse = np.full((B, H, N), -np.inf)
    for h in range(H):
        for b in range(B):
            # a row at or past the batch's length is in no segment
            n = np.arange(N)
            real = n < lens[b]
            M = multiplicity(lens[b], patterns, causal, h) if lens[b] > 0 else np.zeros((0, 0))
            M = np.pad(M, ((0, N - lens[b]), (0, N - lens[b]))) * (real[:, None] & real[None, :])
            S = scale * (q[b, :, h] @ k[b, :, h].T)
            covered = M.sum(axis=1) > 0
            m = np.where(M > 0, S, -np.inf).max(axis=1)
            m = np.where(covered, m, 0.0)
            W = M * np.exp(S - m[:, None])
            den = W.sum(axis=1)
            safe = np.where(covered, den, 1.0)
            o[b, :, h] = np.where(covered[:, None], (W @ v[b, :, h]) / safe[:, None], 0.0)
            lse[b, h] = np.where(covered, m + np.log(safe), -np.inf)
    return o, lse


def multiplicity(N, patterns, causal, h):
    """M_h[q, k]: how many patterns put keys k in the dilated segment of query q (head h)."""
    n = np.arange(N)
    M = np.zeros((N, N))
    for w, r in patterns:
        kept = (n % r) == (h % r)
        same = (n[:, None] // w) == (n[None, :] // w)
        M += kept[:, None] & kept[None, :] & same
    if causal:
        M *= n[None, :] <= n[:, None]
    return M


def pair_count(B, N, H, patterns, causal, lengths=None):
    """Unmasked (query, key) pairs the method evaluates, summed over patterns.

    Per head and pattern: segments of L sparse rows (L = w/r, fewer in a
    shorter last segment), each holding L(L+1)/2 causal or L*L non-causal
    pairs.  With fixed w/r this grows linearly in N ([G] 方法论: linear
    complexity O(Nd)).
    """
    total = 0
    for n_b in _lengths(lengths, B, N):
        for w, r in patterns:
            for h in range(H):
                for s in range(segments(n_b, w)):
                    L = segment_rows(n_b, w, r, h, s).size
                    total += L * (L + 1) // 2 if causal else L * L
    return total

