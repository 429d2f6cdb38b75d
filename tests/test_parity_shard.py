"""GPU parity of sequence shards (needs an MI355X).

One device's share of the sequence-split scheme (the gptget.net LongNet
summary, section 方法论, distributed item): the sequence of total_rows rows is
cut into G shards of N rows; a segment longer than a shard spans devices, and
its sparsified keys and values are exchanged.  Here every device is played by
slices of one tensor on one GPU: each shard's part of the exchange comes from
dla_shard_gather on that shard's slice, the parts of a segment's devices are
stacked in device order (what an all-gather returns), and dla_forward_shard
must reproduce the oracle's result for the whole sequence on the shard's
rows.  Every call goes through the C ABI.
"""
import numpy as np
import pytest

import oracle
from sparse_long_sequence_dilated_amd import dla, inputs
from tests.gpu_util import ORACLE_WORKERS, TOL, check_fwd, normwise, to_device, to_host

pytestmark = pytest.mark.gpu


def _gathered(x, pats, p, N, total, g):
    """[w/N, B, H, N/r, D]: the parts of the devices of shard g's segment."""
    import torch
    w = pats[p][0]
    s = (g * N) // w
    parts = []
    for gd in range(s * w // N, (s + 1) * w // N):
        parts.append(dla.shard_gather(x[:, gd * N:(gd + 1) * N], pats, p, total, gd * N))
    return torch.stack(parts).contiguous()


def _run_shards(tq, tk, tv, pats, causal, scale, N, total):
    import torch
    outs, lses = [], []
    for g in range(total // N):
        ext_k, ext_v = {}, {}
        for p, (w, r) in enumerate(pats):
            if w > N:
                ext_k[p] = _gathered(tk, pats, p, N, total, g)
                ext_v[p] = _gathered(tv, pats, p, N, total, g)
        sl = slice(g * N, (g + 1) * N)
        # outputs start as NaN, so an entry the library never writes cannot pass
        o = _nan_like(tq[:, sl])
        lse = torch.full((tq.shape[0], tq.shape[2], N), float("nan"), device="cuda")
        dla.forward_shard(tq[:, sl], tk[:, sl], tv[:, sl], pats, total, g * N, ext_k, ext_v,
                          causal, scale, out=o, lse=lse)
        outs.append(o)
        lses.append(lse)
    torch.cuda.synchronize()
    return torch.cat(outs, dim=1), torch.cat(lses, dim=2)


def _nan_like(t):
    """A NaN-filled tensor with t's shape and strides (the library's outputs share q's layout)."""
    import torch
    return torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device).fill_(float("nan"))


def test_shard_gather_is_exact():
    import torch
    B, N, H, total = 2, 512, 3, 2048
    pats = ((256, 1), (1024, 4), (2048, 4))
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    x = torch.randn((B, total, H, 64), device="cuda", generator=g).bfloat16()
    for p in (1, 2):
        r = pats[p][1]
        for gd in range(total // N):
            xs = x[:, gd * N:(gd + 1) * N]
            got = dla.shard_gather(xs, pats, p, total, gd * N)
            want = torch.stack([xs[:, (h % r)::r, h, :] for h in range(H)], dim=1)
            assert torch.equal(got, want), (p, gd)


CASES = [
    # (B, total, H, patterns, causal, G)
    (2, 2048, 3, ((256, 1), (1024, 4), (2048, 4)), True, 4),
    (2, 2048, 3, ((256, 1), (1024, 4), (2048, 4)), False, 4),
    (1, 2048, 2, ((256, 1), (1024, 4), (2048, 4)), True, 8),      # N/r = 64: one tile per chunk
    (1, 4096, 3, ((512, 1), (4096, 2)), True, 2),                 # r = 1 local, two-device segment
    (1, 2048, 2, ((2048, 1),), True, 4),                          # one spanning pattern, r = 1
    (1, 2048, 13, ((2048, 4), (1024, 2)), True, 4),               # every pattern spans; uncovered rows
    # drawn at random (local patterns with w | N, spanning ones with w = N 2^k, r | N and
    # N / r a multiple of 128), kept when the planner accepts every shard
    (2, 2048, 3, ((128, 1), (1024, 2)), True, 4),
    (1, 2048, 3, ((1024, 4), (1024, 4), (2048, 2)), True, 2),     # duplicate local pattern
    (1, 1024, 2, ((512, 1),), True, 4),
    (2, 1024, 1, ((512, 2),), False, 4),
    (1, 4096, 4, ((4096, 4), (2048, 1), (2048, 2)), True, 4),
    (1, 4096, 5, ((4096, 2),), False, 4),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}G{c[5]}-"
                         f"{'c' if c[4] else 'nc'}-{'_'.join(f'{w}x{r}' for w, r in c[3])}")
def test_forward_shards_match_whole_sequence_oracle(case):
    B, total, H, pats, causal, G = case
    N = total // G
    seed = sum(ord(ch) for ch in str(case))
    q, k, v = inputs.random_case(seed, B, total, H, "bf16")
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    o, lse = _run_shards(tq, tk, tv, pats, causal, 0.125, N, total)
    o_ref, lse_ref = oracle.forward(q, k, v, pats, causal, 0.125)
    eo, el = check_fwd(to_host(o), to_host(lse), o_ref, lse_ref, "bf16")


@pytest.fixture(scope="module")
def c4_last_shard():
    """C4 split over 8 devices, the last shard (patterns i = 7..9 span 2, 4 and
    8 devices), run once into NaN-filled outputs: (q, k, v, o, lse) on the
    host for the shard's rows."""
    import torch
    wl = inputs.WORKLOADS["C4"]
    total, G = wl.N, 8
    N = total // G
    q, k, v = inputs.workload_inputs(wl)
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    g = G - 1
    ext_k, ext_v = {}, {}
    for p, (w, r) in enumerate(wl.patterns):
        if w > N:
            ext_k[p] = _gathered(tk, wl.patterns, p, N, total, g)
            ext_v[p] = _gathered(tv, wl.patterns, p, N, total, g)
    sl = slice(g * N, (g + 1) * N)
    o = torch.full_like(tq[:, sl], float("nan"))
    lse = torch.full((wl.B, wl.H, N), float("nan"), dtype=torch.float32, device="cuda")
    dla.forward_shard(tq[:, sl], tk[:, sl], tv[:, sl], wl.patterns, total, g * N,
                      ext_k, ext_v, True, wl.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    del tq, tk, tv, ext_k, ext_v
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    out = q, k, v, to_host(o), to_host(lse)
    del o, lse
    torch.cuda.empty_cache()
    return out


@pytest.mark.parametrize("h", range(12))
def test_forward_shard_c4_eight_way_last_shard_full(c4_last_shard, h):
    """Every row of the last of 8 C4 shards against the whole-sequence
    float32 oracle, one head at a time."""
    wl = inputs.WORKLOADS["C4"]
    N = wl.N // 8
    q, k, v, o, lse = c4_last_shard
    hs = slice(h, h + 1)
    o_ref, lse_ref = oracle.forward(q[:, :, hs], k[:, :, hs], v[:, :, hs], wl.patterns, True, wl.scale,
                                    dtype=np.float32, workers=ORACLE_WORKERS, heads=[h])
    rows = slice(wl.N - N, wl.N)
    check_fwd(o[:, :, h], lse[:, h], o_ref[:, rows, 0], lse_ref[:, 0, rows], "bf16",
              f"C4 shard 7/8 head {h}:")


BWD_CASES = [
    # (B, total, H, patterns, causal, G): spanning patterns need N / r % 128 == 0
    (2, 2048, 3, ((256, 1), (1024, 4), (2048, 4)), True, 4),
    (1, 2048, 3, ((256, 1), (1024, 4), (2048, 4)), False, 4),
    (1, 4096, 3, ((512, 1), (4096, 2)), True, 2),
    (1, 2048, 2, ((2048, 1),), True, 4),
    (1, 2048, 13, ((2048, 4), (1024, 2)), True, 4),               # every pattern spans
    (2, 2048, 3, ((128, 1), (1024, 2)), True, 4),                 # drawn at random (as above)
    (1, 2048, 3, ((1024, 4), (1024, 4), (2048, 2)), True, 2),
    (2, 1024, 1, ((512, 2),), False, 4),
    (1, 4096, 4, ((4096, 4), (2048, 1), (2048, 2)), True, 4),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}G{c[5]}-"
                         f"{'c' if c[4] else 'nc'}-{'_'.join(f'{w}x{r}' for w, r in c[3])}")
def test_backward_shards_match_whole_sequence_oracle(case):
    """Each shard's backward, the exchange of the segments' dK/dV summed over
    their devices (a reduce-scatter), then each shard's finish pass."""
    import torch
    B, total, H, pats, causal, G = case
    N = total // G
    seed = 7 + sum(ord(ch) for ch in str(case))
    q, k, v, dout = inputs.random_case(seed, B, total, H, "bf16", count=4)
    tq, tk, tv, tdo = (to_device(x, "bf16") for x in (q, k, v, dout))
    span = [p for p, (w, r) in enumerate(pats) if w > N]
    first = []
    for g in range(G):
        sl = slice(g * N, (g + 1) * N)
        ext_k = {p: _gathered(tk, pats, p, N, total, g) for p in span}
        ext_v = {p: _gathered(tv, pats, p, N, total, g) for p in span}
        o, lse = dla.forward_shard(tq[:, sl], tk[:, sl], tv[:, sl], pats, total, g * N, ext_k, ext_v,
                                   causal, 0.125)
        nan = [_nan_like(tq[:, sl]) for _ in range(3)]
        first.append(dla.backward_shard(tq[:, sl], tk[:, sl], tv[:, sl], o, lse, tdo[:, sl], pats,
                                        total, g * N, ext_k, ext_v, causal, 0.125,
                                        dq=nan[0], dk=nan[1], dv=nan[2]))
    # the exchange: device g of a segment gets the sum over the segment's devices of their parts
    dqs, dks, dvs = [], [], []
    for g in range(G):
        red_k, red_v = {}, {}
        for p in span:
            w = pats[p][0]
            d0 = (g * N) // w * (w // N)
            red_k[p] = sum(first[d][3][p][g - d0] for d in range(d0, d0 + w // N)).contiguous()
            red_v[p] = sum(first[d][4][p][g - d0] for d in range(d0, d0 + w // N)).contiguous()
        dq, dk, dv, _, _, ws = first[g]
        dla.finish_shard(dk, dv, pats, total, g * N, red_k, red_v, ws, causal, 0.125)
        dqs.append(dq)
        dks.append(dk)
        dvs.append(dv)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(q, k, v, pats, causal, 0.125)
    refs = oracle.backward(q, k, v, o_ref, lse_ref, dout, pats, causal, 0.125)
    for name, got, ref in zip(("dq", "dk", "dv"), (dqs, dks, dvs), refs):
        e = normwise(to_host(torch.cat(got, dim=1)), ref)
        print(f"{case} {name}: {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (name, e)
