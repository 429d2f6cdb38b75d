"""Pins of the CPU oracle against things other than itself (CPU only).

Pins used (the pages print no worked numbers, so none is pinned by printed values):
  * hand-derived worked examples (tests/golden/uniform_small.json);
  * the union-softmax brute force on a dense multiplicity matrix;
  * w = N, r = 1 is full attention: torch's scaled_dot_product_attention in fp64
    (the abstract on the gptget.net page calls the method a drop-in replacement
    for standard attention);
  * a single (w, 1) pattern is block-diagonal attention (torch SDPA with a mask);
  * rows no pattern selects: O = 0, LSE = -inf, zero gradients;
  * pattern order invariance and duplicate patterns (LSE + ln 2, O unchanged);
  * backward: central finite differences, torch autograd of an independent
    dense formulation, and SDPA autograd for w = N, r = 1;
  * the work counter against brute-force counting, and its linear growth in N
    (gptget.net page, section 方法论: linear complexity).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_long_sequence_dilated_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, (int, float)):
        return float(x)
    if x == "-inf":
        return -math.inf
    if x == "0":
        return 0.0
    if x.startswith("ln"):
        return math.log(float(x[2:]))
    if "/" in x:
        a, b = x.split("/")
        return float(a) / float(b)
    return float(x)


def _rand(seed, B, N, H, D, count=3):
    g = np.random.default_rng(seed)
    return [g.standard_normal((B, N, H, D)) for _ in range(count)]


PATTERN_SETS = [
    ((8, 1), (16, 2), (32, 4)),
    ((4, 1), (8, 2), (16, 4), (32, 8), (64, 16)),   # r up to 16 > H
    ((16, 2), (32, 4)),                            # no r = 1: some rows uncovered
    ((8, 2), (8, 2), (32, 1)),                     # duplicate pattern
    ((64, 1),),                                    # full attention
    ((12, 3), (24, 6), (48, 3)),                   # non-power-of-2 rates
]


# ---------------------------------------------------------------- golden ----

def test_golden_uniform_examples():
    with open(os.path.join(GOLDEN, "uniform_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        N, H, D = c["N"], c["H"], c["D"]
        q = np.zeros((1, N, H, D))
        k = np.zeros((1, N, H, D))
        v = np.zeros((1, N, H, D))
        for h in range(H):
            v[0, :, h, 0] = [_num(x) for x in c[f"v_head{h}"]]
            if f"q_head{h}" in c:
                q[0, :, h, 0] = [_num(x) for x in c[f"q_head{h}"]]
                k[0, :, h, 0] = [_num(x) for x in c[f"k_head{h}"]]
        pats = [tuple(p) for p in c["patterns"]]
        o, lse = oracle.forward(q, k, v, pats, c["causal"], c["scale"])
        for h in range(H):
            exp_o = np.array([_num(x) for x in c[f"o_head{h}"]])
            exp_lse = np.array([_num(x) for x in c[f"lse_head{h}"]])
            np.testing.assert_allclose(o[0, :, h, 0], exp_o, rtol=1e-13, atol=1e-13, err_msg=c["name"])
            fin = np.isfinite(exp_lse)
            assert np.array_equal(np.isfinite(lse[0, h]), fin), c["name"]
            np.testing.assert_allclose(lse[0, h][fin], exp_lse[fin], rtol=1e-13, atol=1e-13, err_msg=c["name"])


# ------------------------------------------------------------- forward ----

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pats", PATTERN_SETS)
def test_forward_matches_union_softmax_brute_force(pats, causal):
    N = max(w for w, _ in pats)
    N = N * (2 if N <= 32 else 1)
    q, k, v = _rand(hash((pats, causal)) & 0xFFFF, 2, N, 5, 8)
    o, lse = oracle.forward(q, k, v, pats, causal, 0.3)
    ob, lseb = oracle.brute_force_forward(q, k, v, pats, causal, 0.3)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isfinite(lse), np.isfinite(lseb))
    np.testing.assert_allclose(lse[np.isfinite(lse)], lseb[np.isfinite(lseb)], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_full_pattern_is_standard_attention(causal):
    B, N, H, D = 2, 96, 3, 16
    q, k, v = _rand(7, B, N, H, D)
    o, lse = oracle.forward(q, k, v, [(N, 1)], causal, 0.25)
    t = [torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=0.25)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)
    S = 0.25 * torch.einsum("bhqd,bhkd->bhqk", t[0], t[1])
    if causal:
        S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(S, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_single_block_pattern_is_block_diagonal_attention(causal):
    B, N, H, D, w = 1, 64, 2, 8, 16
    q, k, v = _rand(11, B, N, H, D)
    o, _ = oracle.forward(q, k, v, [(w, 1)], causal, 0.5)
    n = torch.arange(N)
    mask = (n[:, None] // w) == (n[None, :] // w)
    if causal:
        mask &= n[None, :] <= n[:, None]
    t = [torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=mask, scale=0.5)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)


def test_single_dilated_pattern_is_attention_on_gathered_rows():
    # (w, r) for head h: rows h mod r, h mod r + r, ... of each segment, attended densely.
    B, N, H, D, w, r = 1, 64, 3, 8, 32, 4
    q, k, v = _rand(12, B, N, H, D)
    o, lse = oracle.forward(q, k, v, [(w, r)], True, 0.5)
    for h in range(H):
        for s in range(N // w):
            rows = list(range(s * w + h % r, (s + 1) * w, r))
            t = [torch.from_numpy(x[:, rows, h]).unsqueeze(1) for x in (q, k, v)]
            ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True, scale=0.5)
            np.testing.assert_allclose(o[0, rows, h], ref[0, 0].numpy(), rtol=1e-12, atol=1e-12)
        kept = np.zeros(N, bool)
        kept[h % r::r] = True
        assert np.all(o[0, ~kept, h] == 0.0) and np.all(np.isneginf(lse[0, h, ~kept]))


def test_uncovered_rows_are_zero_with_neg_inf_lse():
    q, k, v = _rand(3, 2, 32, 3, 8)
    o, lse = oracle.forward(q, k, v, [(16, 2), (32, 4)], True, 0.3)
    for h in range(3):
        unc = (np.arange(32) % 2) != (h % 2)
        assert np.all(o[:, unc, h] == 0.0)
        assert np.all(np.isneginf(lse[:, h, unc]))
        assert np.all(np.isfinite(lse[:, h, ~unc]))


def test_pattern_order_invariance_and_duplicates():
    q, k, v = _rand(5, 1, 64, 4, 8)
    pats = [(8, 1), (16, 2), (64, 8)]
    o1, l1 = oracle.forward(q, k, v, pats, True, 0.3)
    o2, l2 = oracle.forward(q, k, v, pats[::-1], True, 0.3)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)
    od, ld = oracle.forward(q, k, v, [(16, 2), (16, 2)], True, 0.3)
    os_, ls = oracle.forward(q, k, v, [(16, 2)], True, 0.3)
    np.testing.assert_allclose(od, os_, rtol=1e-13, atol=1e-13)
    fin = np.isfinite(ls)
    np.testing.assert_allclose(ld[fin], ls[fin] + math.log(2.0), rtol=1e-13, atol=1e-13)


def test_forward_rows_matches_forward():
    q, k, v = _rand(9, 2, 128, 5, 8)
    pats = [(16, 1), (32, 2), (64, 4), (128, 8)]
    o, lse = oracle.forward(q, k, v, pats, True, 0.3)
    rows = np.array([0, 1, 7, 31, 32, 63, 100, 127])
    for b in range(2):
        for h in range(5):
            orow, lrow = oracle.forward_rows(q, k, v, pats, True, 0.3, b, h, rows)
            np.testing.assert_allclose(orow, o[b, rows, h], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lrow, lse[b, h, rows], rtol=1e-12, atol=1e-12)


def test_single_head_slices_match_the_brute_force_heads():
    """forward on one head's slice, with `heads` naming that head, gives the
    head's result: its row offsets follow the named head (h mod r), checked
    against the union-softmax brute force on all heads (rates 3 and 4 make
    every head's offset set differ)."""
    q, k, v = _rand(31, 2, 96, 5, 8)
    pats = [(12, 1), (24, 3), (48, 4), (96, 12)]
    ob, lb = oracle.brute_force_forward(q, k, v, pats, True, 0.3)
    for h in range(5):
        sl = slice(h, h + 1)
        o, lse = oracle.forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], pats, True, 0.3, heads=[h],
                                workers=2)
        np.testing.assert_allclose(o[:, :, 0], ob[:, :, h], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[:, 0], lb[:, h], rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, pats, True, 0.3, heads=[0])


def test_float32_and_threaded_paths_agree_with_float64():
    wl = inputs.WORKLOADS["C1"]
    q, k, v = inputs.draw((1, 512, 4, 64), 1, 3, "f32")
    pats = [(128, 1), (256, 2), (512, 4)]
    o64, l64 = oracle.forward(q, k, v, pats, False, wl.scale)
    o32, l32 = oracle.forward(q, k, v, pats, False, wl.scale, dtype=np.float32, workers=4)
    assert o32.dtype == np.float32
    assert np.abs(o32 - o64).max() / np.abs(o64).max() < 2e-6
    assert np.abs(l32 - l64).max() / np.abs(l64).max() < 2e-6


# ------------------------------------------------------------ backward ----

def _loss(q, k, v, dout, pats, causal, scale):
    o, _ = oracle.forward(q, k, v, pats, causal, scale)
    return float((o * dout).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pats", [((4, 1), (8, 2), (16, 4)), ((8, 2), (16, 4)), ((6, 3), (12, 1))])
def test_backward_matches_finite_differences(pats, causal):
    N = 16 if max(w for w, _ in pats) <= 16 else 32
    N = 24 if pats == ((6, 3), (12, 1)) else N
    q, k, v, dout = _rand(21, 1, N, 2, 4, count=4)
    o, lse = oracle.forward(q, k, v, pats, causal, 0.7)
    grads = oracle.backward(q, k, v, o, lse, dout, pats, causal, 0.7)
    g = np.random.default_rng(5)
    eps = 1e-6
    for which in range(3):
        for _ in range(3):
            d = g.standard_normal(q.shape)
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p = [a + eps * d if i == which else a for i, a in enumerate(args_p)]
            args_m = [a - eps * d if i == which else a for i, a in enumerate(args_m)]
            fd = (_loss(*args_p, dout, pats, causal, 0.7) - _loss(*args_m, dout, pats, causal, 0.7)) / (2 * eps)
            an = float((grads[which] * d).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def _torch_dense_union(q, k, v, pats, causal, scale):
    """Independent dense formulation: multiplicity matrix built by enumerating segments."""
    B, N, H, D = q.shape
    outs = []
    for h in range(H):
        M = torch.zeros(N, N, dtype=torch.float64)
        for w, r in pats:
            for s in range(-(-N // w)):                 # a last, shorter segment keeps its rows
                rows = list(range(s * w + h % r, min((s + 1) * w, N), r))
                for i, a in enumerate(rows):
                    for j, c in enumerate(rows):
                        if causal and j > i:
                            continue
                        M[a, c] += 1.0
        S = scale * q[:, :, h] @ k[:, :, h].transpose(1, 2)
        S = torch.where(M > 0, S, torch.full_like(S, -math.inf))
        logw = S + torch.log(torch.clamp(M, min=1e-300))
        prob = torch.softmax(logw, dim=-1)
        prob = torch.nan_to_num(prob, nan=0.0)
        outs.append(prob @ v[:, :, h])
    return torch.stack(outs, dim=2)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_autograd_of_dense_union(causal):
    pats = [(8, 1), (16, 2), (32, 4), (32, 8)]
    q, k, v, dout = _rand(31, 2, 32, 3, 8, count=4)
    o, lse = oracle.forward(q, k, v, pats, causal, 0.4)
    dq, dk, dv = oracle.backward(q, k, v, o, lse, dout, pats, causal, 0.4)
    t = [torch.from_numpy(x).requires_grad_(True) for x in (q, k, v)]
    ot = _torch_dense_union(*t, pats, causal, 0.4)
    np.testing.assert_allclose(ot.detach().numpy(), o, rtol=1e-12, atol=1e-12)
    ot.backward(torch.from_numpy(dout))
    for mine, ref in zip((dq, dk, dv), t):
        np.testing.assert_allclose(mine, ref.grad.numpy(), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_full_pattern_matches_sdpa_autograd(causal):
    B, N, H, D = 1, 64, 2, 16
    q, k, v, dout = _rand(41, B, N, H, D, count=4)
    o, lse = oracle.forward(q, k, v, [(N, 1)], causal, 0.25)
    dq, dk, dv = oracle.backward(q, k, v, o, lse, dout, [(N, 1)], causal, 0.25)
    t = [torch.from_numpy(x).permute(0, 2, 1, 3).contiguous().requires_grad_(True) for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=0.25)
    ref.backward(torch.from_numpy(dout).permute(0, 2, 1, 3))
    for mine, r in zip((dq, dk, dv), t):
        np.testing.assert_allclose(mine, r.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-11)


def test_backward_uncovered_rows_have_zero_gradient():
    q, k, v, dout = _rand(51, 1, 32, 2, 8, count=4)
    pats = [(16, 2)]
    o, lse = oracle.forward(q, k, v, pats, True, 0.3)
    dq, dk, dv = oracle.backward(q, k, v, o, lse, dout, pats, True, 0.3)
    for h in range(2):
        unc = (np.arange(32) % 2) != (h % 2)
        for g in (dq, dk, dv):
            assert np.all(g[:, unc, h] == 0.0)


# ------------------------------------------------------- work and rows ----

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pats", PATTERN_SETS)
def test_pair_count_matches_brute_force(pats, causal):
    N, H = math.lcm(*[w for w, _ in pats]), 5
    N *= max(1, 128 // N)
    counted = sum(oracle.multiplicity(N, pats, causal, h).sum() for h in range(H))
    assert oracle.pair_count(2, N, H, pats, causal) == 2 * counted


def test_work_grows_linearly_with_sequence_length():
    # Geometric schedule w = 2048 * 2^i, r = 2^i: every segment has L = 2048 rows,
    # so pairs per token stay below (L + 1) per head however long the sequence is.
    per_token = []
    for count in range(1, 11):
        N = 2048 * 2 ** (count - 1)
        pats = inputs.geometric_patterns(2048, 2, count)
        per_token.append(oracle.pair_count(1, N, 1, pats, True) / N)
    assert all(x < 2049 for x in per_token)
    assert all(b > a for a, b in zip(per_token, per_token[1:]))
    dense_c3 = 32768 * 32769 // 2
    assert oracle.pair_count(1, 32768, 1, inputs.WORKLOADS["C3"].patterns, True) * 8 < dense_c3


@pytest.mark.parametrize("w,r", [(8, 1), (16, 4), (64, 16), (48, 3), (32, 32)])
def test_row_map_properties(w, r):
    N = 192 if w == 48 else 128
    for h in range(7):
        m = oracle.row_map(N, w, r, h)
        assert m.shape == (N // r,)
        assert np.all(np.diff(m) > 0)
        assert np.all(m % r == h % r)
        assert m.min() >= 0 and m.max() < N
        L = w // r
        seg = np.repeat(np.arange(N // w), L)
        assert np.all(m // w == seg)
        kept = (np.arange(N) % r) == (h % r)
        assert np.array_equal(np.sort(m), np.nonzero(kept)[0])


# ------------------------------------------- a shorter last segment ----
# The pages are silent on N % w != 0; the reading taken is that the last
# segment keeps the rows that remain (one segment of N rows when w > N).

CLAMPED = [((16, 2), (64, 4)), ((12, 1), (24, 3)), ((48, 1),), ((16, 1), (32, 2), (64, 8))]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pats", CLAMPED)
def test_clamped_forward_matches_union_softmax_brute_force(pats, causal):
    q, k, v = _rand(hash((pats, causal, 40)) & 0xFFFF, 2, 40, 5, 8)
    o, lse = oracle.forward(q, k, v, pats, causal, 0.3)
    ob, lseb = oracle.brute_force_forward(q, k, v, pats, causal, 0.3)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isfinite(lse), np.isfinite(lseb))
    np.testing.assert_allclose(lse[np.isfinite(lse)], lseb[np.isfinite(lseb)], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_segment_longer_than_sequence_is_standard_attention(causal):
    B, N, H, D = 1, 40, 2, 16
    q, k, v = _rand(17, B, N, H, D)
    o, _ = oracle.forward(q, k, v, [(64, 1)], causal, 0.25)
    t = [torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=0.25)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("pats", CLAMPED)
def test_causal_result_equals_padded_sequence(pats):
    # Under the causal mask, rows appended after the sequence are never keys
    # of a real row, so padding to a multiple of every w with arbitrary rows
    # leaves the real rows' result unchanged.
    N = 40
    Np = math.lcm(*[w for w, _ in pats])
    Np *= -(-N // Np)
    q, k, v = _rand(61, 2, Np, 3, 8)
    o_pad, lse_pad = oracle.forward(q, k, v, pats, True, 0.35)
    o, lse = oracle.forward(q[:, :N], k[:, :N], v[:, :N], pats, True, 0.35)
    np.testing.assert_allclose(o, o_pad[:, :N], rtol=1e-12, atol=1e-12)
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(lse_pad[:, :, :N]))
    np.testing.assert_allclose(lse[fin], lse_pad[:, :, :N][fin], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pats", CLAMPED[:2])
def test_clamped_backward_matches_autograd_of_dense_union(pats, causal):
    q, k, v, dout = _rand(71, 2, 40, 3, 8, count=4)
    o, lse = oracle.forward(q, k, v, pats, causal, 0.4)
    dq, dk, dv = oracle.backward(q, k, v, o, lse, dout, pats, causal, 0.4)
    t = [torch.from_numpy(x).requires_grad_(True) for x in (q, k, v)]
    ot = _torch_dense_union(*t, pats, causal, 0.4)
    np.testing.assert_allclose(ot.detach().numpy(), o, rtol=1e-12, atol=1e-12)
    ot.backward(torch.from_numpy(dout))
    for mine, ref in zip((dq, dk, dv), t):
        np.testing.assert_allclose(mine, ref.grad.numpy(), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pats", CLAMPED)
def test_clamped_pair_count_matches_brute_force(pats, causal):
    N, H = 40, 5
    counted = sum(oracle.multiplicity(N, pats, causal, h).sum() for h in range(H))
    assert oracle.pair_count(2, N, H, pats, causal) == 2 * counted


@pytest.mark.parametrize("w,r", [(16, 2), (64, 4), (12, 3), (48, 1)])
def test_clamped_row_map_covers_each_kept_row_once(w, r):
    N = 40
    for h in range(6):
        m = oracle.row_map(N, w, r, h)
        assert m.shape == (-(-N // r),)
        valid = m[m >= 0]
        assert np.array_equal(np.sort(valid), np.arange(N)[np.arange(N) % r == h % r])
        # sparse entry s*(w/r) + a of a row in segment s
        L = w // r
        for i, n in enumerate(m):
            if n >= 0:
                assert i // L == n // w and n == (i // L) * w + h % r + (i % L) * r


# ---------------------------------------------- batches of different lengths ----
# Batch b is the sequence of its first lengths[b] rows; the rows after it are
# padding (output 0, log-sum-exp -inf, zero gradients).

VARLEN = [(40, 17, 0, 33), (40, 40, 1, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pats", [((16, 2), (64, 4)), ((12, 1), (24, 3))])
@pytest.mark.parametrize("lens", VARLEN)
def test_varlen_forward_matches_union_softmax_brute_force(pats, causal, lens):
    N = max(max(lens), 40)
    q, k, v = _rand(hash((pats, causal, lens)) & 0xFFFF, len(lens), N, 3, 8)
    o, lse = oracle.forward(q, k, v, pats, causal, 0.3, lengths=lens)
    ob, lseb = oracle.brute_force_forward(q, k, v, pats, causal, 0.3, lengths=lens)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isfinite(lse), np.isfinite(lseb))
    np.testing.assert_allclose(lse[np.isfinite(lse)], lseb[np.isfinite(lseb)], rtol=1e-12, atol=1e-12)
    for b, n_b in enumerate(lens):
        assert np.all(o[b, n_b:] == 0.0) and np.all(lse[b, :, n_b:] == -np.inf)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_backward_matches_autograd_of_dense_union(causal):
    pats = [(16, 2), (64, 4)]
    lens = (40, 23)
    q, k, v, dout = _rand(81, 2, 40, 3, 8, count=4)
    o, lse = oracle.forward(q, k, v, pats, causal, 0.4, lengths=lens)
    dq, dk, dv = oracle.backward(q, k, v, o, lse, dout, pats, causal, 0.4, lengths=lens)
    for b, n_b in enumerate(lens):
        t = [torch.from_numpy(x[b:b + 1, :n_b].copy()).requires_grad_(True) for x in (q, k, v)]
        ot = _torch_dense_union(*t, pats, causal, 0.4)
        np.testing.assert_allclose(ot.detach().numpy()[0], o[b, :n_b], rtol=1e-12, atol=1e-12)
        ot.backward(torch.from_numpy(dout[b:b + 1, :n_b].copy()))
        for mine, ref in zip((dq, dk, dv), t):
            np.testing.assert_allclose(mine[b, :n_b], ref.grad.numpy()[0], rtol=1e-11, atol=1e-11)
            assert np.all(mine[b, n_b:] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_pair_count_matches_brute_force(causal):
    pats = ((16, 2), (64, 4), (12, 1))
    lens = (40, 17, 0, 33)
    want = sum(oracle.multiplicity(n_b, pats, causal, h).sum() for n_b in lens if n_b
               for h in range(5))
    assert oracle.pair_count(len(lens), 40, 5, pats, causal, lengths=lens) == want


def _hops_to_connect(N, pats, heads, causal):
    """Fewest attention hops after which every row reaches every (earlier) row,
    a hop going from a query to a key that some head and pattern let it see
    (the heads are mixed between layers); None if some pair never connects."""
    A = np.zeros((N, N), dtype=bool)
    for h in range(heads):
        A |= oracle.multiplicity(N, pats, causal, h) > 0
    target = np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)
    R, hops = A.copy(), 1
    while not R[target].all():
        grown = ((R.astype(np.int64) @ A.astype(np.int64)) > 0) | R
        if np.array_equal(grown, R):
            return None
        R, hops = grown, hops + 1
    return hops


@pytest.mark.parametrize("w0,levels", [(2, 5), (4, 6), (8, 6)])
def test_geometric_patterns_connect_rows_in_logarithmic_hops(w0, levels):
    """gptget.net page, 方法详解 (sixth item) and the darcstar.tech commentary:
    local attention plus dilated global sampling keeps the path between any
    two tokens logarithmic.  With the geometric schedule (w0 2^i, 2^i) over
    N = w0 2^(levels-1) and every head offset present, every row reaches
    every other row within log2(N / w0) + 1 hops, while the local pattern
    alone never leaves its segment."""
    N = w0 * 2 ** (levels - 1)
    pats = inputs.geometric_patterns(w0, 2, levels)
    hops = _hops_to_connect(N, pats, 2 ** (levels - 1), causal=False)
    assert hops is not None and hops <= levels
    assert _hops_to_connect(N, [(w0, 1)], 1, causal=False) is None
    # under the causal mask a row cannot reach an earlier row that a later
    # key between them never sees: e.g. row w0 (first of its block) and row w0-1
    assert _hops_to_connect(N, pats, 2 ** (levels - 1), causal=True) is None


@pytest.mark.parametrize("causal", [False, True])
def test_backward_dq_rows_match_full_backward(causal):
    """The row-at-a-time dQ equals the full backward's dQ rows (including
    uncovered rows, cut-short segments and duplicate patterns)."""
    pats = [(8, 1), (16, 2), (24, 4), (8, 1), (20, 5)]
    q, k, v, dout = _rand(61, 2, 45, 3, 8, count=4)
    o, lse = oracle.forward(q, k, v, pats, causal, 0.35)
    dq, _, _ = oracle.backward(q, k, v, o, lse, dout, pats, causal, 0.35)
    rows = np.arange(45)
    for b in range(2):
        for h in range(3):
            got = oracle.backward_dq_rows(q, k, v, dout, pats, causal, 0.35, b, h, rows)
            np.testing.assert_allclose(got, dq[b, :, h], rtol=1e-11, atol=1e-12)
