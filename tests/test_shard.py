"""Sequence shards on the CPU: validation, workspace sizes and pair counts.

A shard is one device's piece of a sequence split along its length (the
gptget.net LongNet summary, section 方法论, distributed item).  Its pair count
is pinned to the oracle's multiplicity matrix restricted to the shard's query
rows, and the counts of all shards must add up to the whole sequence's.
"""
import numpy as np
import pytest

import oracle
from sparse_long_sequence_dilated_amd import dla

PATS = ((256, 1), (1024, 4), (2048, 4))   # total 2048: spanning for N < 1024 / < 2048
TOTAL = 2048


def _align(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("causal", [True, False])
def test_shard_pair_counts_match_oracle_and_add_up(causal):
    B, H = 2, 3
    whole = dla.pair_count(PATS, causal, B, TOTAL, H)
    M = [oracle.multiplicity(TOTAL, PATS, causal, h) for h in range(H)]
    for G in (1, 2, 4, 8):
        N = TOTAL // G
        got = [dla.pair_count_shard(PATS, causal, B, N, H, TOTAL, g * N) for g in range(G)]
        for g in range(G):
            want = B * sum(int(m[g * N:(g + 1) * N].sum()) for m in M)
            assert got[g] == want, (G, g)
        assert sum(got) == whole


def test_shard_workspace_follows_closed_form():
    B, H = 2, 3
    for G in (1, 2, 4, 8):
        N = TOTAL // G
        ws, _ = dla.plan_check_shard(PATS, True, 0.125, B, N, H, TOTAL, (G - 1) * N)
        # partial O and LSE of every pattern but the first r == 1 one, over the shard's rows
        exp = sum(_align(B * H * (N // r) * 64 * 2) + _align(B * H * (N // r) * 4)
                  for i, (w, r) in enumerate(PATS) if i != 0)
        assert ws == exp


@pytest.mark.parametrize("pats,N,total,start,dtype,code", [
    (PATS, 512, 2048, 256, dla.DLA_BF16, dla.DLA_E_INVALID),          # start not a multiple of N
    (PATS, 512, 2048, 2048, dla.DLA_BF16, dla.DLA_E_INVALID),         # start past the end
    (PATS, 512, 2048, -512, dla.DLA_BF16, dla.DLA_E_INVALID),
    (PATS, 768, 2048, 0, dla.DLA_BF16, dla.DLA_E_INVALID),            # N does not divide total
    (((768, 1),), 512, 1536, 0, dla.DLA_BF16, dla.DLA_E_UNSUPPORTED), # spanning w not a multiple of N
    (((768, 1),), 1024, 3072, 0, dla.DLA_BF16, dla.DLA_E_UNSUPPORTED),  # local w does not divide N
    (((2048, 8),), 256, 2048, 0, dla.DLA_BF16, dla.DLA_E_UNSUPPORTED),  # N / r = 32 < 64 rows
    (((2048, 512),), 256, 2048, 0, dla.DLA_BF16, dla.DLA_E_UNSUPPORTED),  # r does not divide N
    (((4096, 1),), 512, 2048, 0, dla.DLA_BF16, dla.DLA_E_UNSUPPORTED),  # w beyond the sequence
    (PATS, 512, 2048, 0, dla.DLA_F32, dla.DLA_E_UNSUPPORTED),         # shards are bf16 only
])
def test_plan_check_shard_rejects(pats, N, total, start, dtype, code):
    assert dla.plan_check_shard_code(pats, True, 0.125, 1, N, 2, total, start, dtype=dtype) == code
    assert dla.lib().dla_last_error()


def test_plan_check_shard_accepts_and_null_shard_is_invalid():
    assert dla.plan_check_shard_code(PATS, True, 0.125, 1, 512, 2, 2048, 1536) == dla.DLA_OK
    d = dla.make_desc(PATS, True, 0.125)
    s = dla.make_shape(1, 512, 2, 64, dla.DLA_BF16)
    assert dla.lib().dla_plan_check_shard(d, s, None, None, None) == dla.DLA_E_INVALID


def test_whole_sequence_as_one_shard_equals_the_plain_plan():
    for causal in (True, False):
        assert dla.pair_count_shard(PATS, causal, 1, TOTAL, 2, TOTAL, 0) == \
            dla.pair_count(PATS, causal, 1, TOTAL, 2)
        ws_f, _ = dla.plan_check(PATS, causal, 0.125, 1, TOTAL, 2)
        assert dla.plan_check_shard(PATS, causal, 0.125, 1, TOTAL, 2, TOTAL, 0)[0] == ws_f


def test_backward_shard_needs_128_row_parts():
    # N / r = 64 for the spanning pattern: the forward accepts it, the backward does not
    pats = ((256, 1), (2048, 4))
    d = dla.make_desc(pats, True, 0.125)
    s = dla.make_shape(1, 256, 2, 64, dla.DLA_BF16)
    sh = dla.Shard(2048, 1792)
    assert dla.plan_check_shard_code(pats, True, 0.125, 1, 256, 2, 2048, 1792) == dla.DLA_OK
    L = dla.lib()
    rc = L.dla_backward_shard(d, s, sh, *([None] * 14), 0, None)
    assert rc == dla.DLA_E_UNSUPPORTED
    rc = L.dla_shard_finish(d, s, sh, None, None, None, None, None, 0, None)
    assert rc == dla.DLA_E_UNSUPPORTED


def test_shard_backward_workspace_holds_partials_and_one_segment():
    B, H, N = 2, 3, 512
    _, wb = dla.plan_check_shard(PATS, True, 0.125, B, N, H, TOTAL, 0)
    exp = _align(B * N * H * 8)
    for w, r in PATS:
        exp += 3 * _align(B * H * (N // r) * 64 * 4)
    lk = max(w // r for w, r in PATS if w > N)
    rows = B * H * lk
    for nbytes in (rows * 128, rows * 128, rows * 8, rows * 128, rows * 128, rows * 256, rows * 256):
        exp += _align(nbytes)
    assert wb == exp
