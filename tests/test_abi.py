"""The C ABI boundary on the CPU: symbols, validation, workspace sizes, work count.

No compute call is made here (there is no GPU); dla_plan_check and
dla_pair_count are host-only.  The planner is also rebuilt with g++ under
the address and undefined-behaviour sanitizers and driven by a C harness.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from sparse_long_sequence_dilated_amd import dla, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dla.h")
CSRC = os.path.join(ROOT, "sparse_long_sequence_dilated_amd", "csrc")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(dla_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert set(names) == set(dla.EXPORTS), names
    lib = dla.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", dla.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(dla_\w+)", out))
    assert set(names) <= exported


def test_strerror_texts():
    lib = dla.lib()
    for code in (0, -1, -2, -3, -4):
        assert lib.dla_strerror(code)
    assert b"unknown" in lib.dla_strerror(-99)


C3 = inputs.WORKLOADS["C3"]


@pytest.mark.parametrize("kwargs,code", [
    (dict(patterns=[]), dla.DLA_E_INVALID),
    (dict(patterns=[(64, 1)] * 17), dla.DLA_E_INVALID),
    (dict(patterns=[(0, 1)]), dla.DLA_E_INVALID),
    (dict(patterns=[(64, 0)]), dla.DLA_E_INVALID),
    (dict(patterns=[(64, -2)]), dla.DLA_E_INVALID),
    (dict(patterns=[(64, 3)]), dla.DLA_E_UNSUPPORTED),       # r does not divide w
    (dict(scale=float("nan")), dla.DLA_E_INVALID),
    (dict(scale=float("inf")), dla.DLA_E_INVALID),
    (dict(scale=0.0), dla.DLA_E_INVALID),
    (dict(scale=-0.1), dla.DLA_E_INVALID),
    (dict(D=128), dla.DLA_E_UNSUPPORTED),
    (dict(dtype=7), dla.DLA_E_UNSUPPORTED),
    (dict(N=0), dla.DLA_E_INVALID),
    (dict(B=-1), dla.DLA_E_INVALID),
    (dict(strides=(256 * 2 * 64, 2 * 64, 60)), dla.DLA_E_INVALID),   # misaligned rows
    (dict(strides=(256 * 2 * 64, 0, 64)), dla.DLA_E_INVALID),
    (dict(causal=2), dla.DLA_E_INVALID),
])
def test_plan_check_rejects(kwargs, code):
    args = dict(patterns=[(64, 1), (128, 2)], causal=True, scale=0.125, B=1, N=256, H=2, D=64,
                dtype=dla.DLA_BF16, strides=None)
    args.update(kwargs)
    causal = args.pop("causal")
    if causal == 2:
        d = dla.make_desc(args["patterns"], True, args["scale"])
        d.causal = 2
        s = dla.make_shape(args["B"], args["N"], args["H"], args["D"], args["dtype"])
        rc = dla.lib().dla_plan_check(d, s, None, None)
    else:
        rc = dla.plan_check_code(args.pop("patterns"), causal, args.pop("scale"), **args)
    assert rc == code
    assert dla.lib().dla_last_error()


def test_segments_cut_short_are_valid():
    # w that does not divide N, and w > N: the last segment keeps the rows that remain
    for pats in ([(96, 1)], [(512, 1)], [(96, 1), (512, 4)], [(100, 4)]):
        assert dla.plan_check_code(pats, True, 0.125, 1, 256, 2) == dla.DLA_OK


@pytest.mark.parametrize("pats", [((96, 1),), ((512, 1),), ((96, 1), (512, 4)), ((100, 4), (48, 3)),
                                  ((3000, 2),)])
@pytest.mark.parametrize("causal", [True, False])
def test_pair_count_cut_short_segments_matches_oracle(pats, causal):
    for N in (256, 1000, 2049):
        assert dla.pair_count(pats, causal, 2, N, 7) == oracle.pair_count(2, N, 7, pats, causal)


def test_workspace_cut_short_segments_uses_ceil_rows():
    # N / r rounded up: the sparse index of row n stays n // r
    N, B, H = 1000, 2, 3
    ws_f, ws_b = dla.plan_check([(96, 1), (510, 3)], True, 0.125, B, N, H)
    rows = B * H * (-(-N // 3))
    assert ws_f == _align(rows * 64 * 2) + _align(rows * 4)
    assert ws_b == _align(B * N * H * 8) + 3 * _align(B * H * N * 64 * 4) + 3 * _align(rows * 64 * 4)


def test_empty_batch_and_heads_are_valid():
    assert dla.plan_check_code([(64, 1)], True, 0.125, 0, 256, 2) == dla.DLA_OK
    assert dla.plan_check_code([(64, 1)], True, 0.125, 1, 256, 0, strides=(256 * 64, 64, 64)) == dla.DLA_OK


def _align(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_workspace_sizes_follow_closed_forms(name):
    wl = inputs.WORKLOADS[name]
    code = dla.DLA_F32 if wl.dtype == "f32" else dla.DLA_BF16
    eb = 4 if wl.dtype == "f32" else 2
    ws_f, ws_b = dla.plan_check(wl.patterns, wl.causal, wl.scale, wl.B, wl.N, wl.H, 64, code)
    # every pattern but the first r == 1 one keeps partial O_p [B,H,N/r,64] and LSE_p [B,H,N/r]
    exp_f = 0
    for i, (w, r) in enumerate(wl.patterns):
        if i == 0:
            continue
        rows = wl.B * wl.H * (wl.N // r)
        exp_f += _align(rows * 64 * eb) + _align(rows * 4)
    # backward: (LSE*log2e, D) pairs [B,H,N]; with several patterns, fp32
    # partial dQ, dK, dV [B,H,N/r,64] per pattern
    exp_b = _align(wl.B * wl.N * wl.H * 8)
    if len(wl.patterns) > 1:
        for w, r in wl.patterns:
            exp_b += 3 * _align(wl.B * wl.H * (wl.N // r) * 64 * 4)
    assert (ws_f, ws_b) == (exp_f, exp_b)


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_pair_count_matches_oracle(name):
    wl = inputs.WORKLOADS[name]
    assert dla.pair_count(wl.patterns, wl.causal, wl.B, wl.N, wl.H) == \
        oracle.pair_count(wl.B, wl.N, wl.H, wl.patterns, wl.causal)


def test_pair_count_small_cases_match_brute_force():
    for pats, causal in [([(8, 1), (16, 2)], True), ([(12, 3), (24, 6)], False), ([(32, 32)], True)]:
        N, H = 96 if any(w in (12, 24) for w, _ in pats) else 64, 5
        counted = sum(oracle.multiplicity(N, pats, causal, h).sum() for h in range(H))
        assert dla.pair_count(pats, causal, 3, N, H) == 3 * counted


HARNESS = r"""
#include <math.h>
#include <stdio.h>
#include <string.h>
#include "dla.h"
static int expect(int got, int want, const char* what) {
  if (got != want) { printf("FAIL %s: got %d want %d (%s)\n", what, got, want, dla_last_error()); return 1; }
  return 0;
}
int main(void) {
  int bad = 0;
  dla_pattern pats[17];
  for (int i = 0; i < 17; ++i) { pats[i].w = 2048 << (i % 5); pats[i].r = 1 << (i % 5); }
  dla_desc d = {5, pats, 1, 0.125f};
  dla_shape s = {2, 32768, 12, 64, DLA_BF16, 32768 * 12 * 64, 12 * 64, 64};
  size_t wf = 0, wb = 0;
  bad += expect(dla_plan_check(&d, &s, &wf, &wb), DLA_OK, "C5");
  if (wf == 0 || wb == 0) { printf("FAIL workspace zero\n"); bad++; }
  bad += expect(dla_plan_check(NULL, &s, &wf, &wb), DLA_E_INVALID, "null desc");
  bad += expect(dla_plan_check(&d, NULL, &wf, &wb), DLA_E_INVALID, "null shape");
  d.num_patterns = 17; bad += expect(dla_plan_check(&d, &s, NULL, NULL), DLA_E_INVALID, "17 patterns");
  d.num_patterns = 5; d.patterns = NULL; bad += expect(dla_plan_check(&d, &s, NULL, NULL), DLA_E_INVALID, "null patterns");
  d.patterns = pats; d.scale = NAN; bad += expect(dla_plan_check(&d, &s, NULL, NULL), DLA_E_INVALID, "nan");
  d.scale = 0.125f; s.N = 32768 + 64; bad += expect(dla_plan_check(&d, &s, NULL, NULL), DLA_OK, "last segment cut short");
  s.N = 32768; s.D = 32; bad += expect(dla_plan_check(&d, &s, NULL, NULL), DLA_E_UNSUPPORTED, "D");
  s.D = 64; s.dtype = 5; bad += expect(dla_plan_check(&d, &s, NULL, NULL), DLA_E_UNSUPPORTED, "dtype");
  s.dtype = DLA_F32; s.stride_h = 4; bad += expect(dla_plan_check(&d, &s, NULL, NULL), DLA_E_INVALID, "stride");
  s.stride_h = 64;
  int64_t pairs = 0;
  bad += expect(dla_pair_count(&d, &s, &pairs), DLA_OK, "pairs");
  if (pairs != (int64_t)2 * 12 * 31 * 2048 * 2049 / 2) { printf("FAIL pairs %lld\n", (long long)pairs); bad++; }
  bad += expect(dla_pair_count(&d, &s, NULL), DLA_E_INVALID, "pairs null");
  /* huge problem: sizes must not overflow */
  s.B = 64; s.N = 1 << 30; s.H = 64; s.stride_b = (int64_t)s.N * 64 * 64; s.stride_n = 64 * 64;
  pats[0].w = 1 << 30; pats[0].r = 1 << 19; d.num_patterns = 1;
  /* 64 dilated rows of r = 2^19 and 8 KB each span more than 2 GiB: refused */
  bad += expect(dla_plan_check(&d, &s, &wf, &wb), DLA_E_UNSUPPORTED, "huge span");
  pats[0].r = 1 << 4;   /* 2^26-row segments: 2^64 pairs, refused */
  bad += expect(dla_plan_check(&d, &s, &wf, &wb), DLA_E_UNSUPPORTED, "huge pairs");
  pats[0].r = 1 << 10;
  bad += expect(dla_plan_check(&d, &s, &wf, &wb), DLA_OK, "huge");
  /* one pattern: the backward workspace is the (LSE, D) pairs, 8 bytes per row */
  if (wb != (size_t)64 * (1u << 30) * 64 * 8) { printf("FAIL huge ws %zu\n", wb); bad++; }
  printf(bad ? "FAILED %d\n" : "ALL OK\n", bad);
  return bad != 0;
}
"""


def test_planner_under_sanitizers(tmp_path):
    src = tmp_path / "harness.c"
    src.write_text(HARNESS)
    exe = tmp_path / "harness"
    cmd = ["g++", "-x", "c++", str(src), "-x", "c++", os.path.join(CSRC, "dla_plan.cpp"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-std=c++17", "-g", "-O1",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True,
                         env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ALL OK" in res.stdout


def test_geometric_workloads_have_linear_work():
    c3, c4 = inputs.WORKLOADS["C3"], inputs.WORKLOADS["C4"]
    p3 = dla.pair_count(c3.patterns, True, 1, c3.N, 12) / (c3.N * 12)
    p4 = dla.pair_count(c4.patterns, True, 1, c4.N, 12) / (c4.N * 12)
    assert 1900 < p3 < p4 < 2049
    assert np.isclose(p3, 1024.5 * sum(2.0 ** -i for i in range(5)))


@pytest.mark.parametrize("causal", [True, False])
def test_pair_count_varlen_matches_oracle(causal):
    pats = ((256, 1), (512, 2), (2048, 4))
    lens = (1000, 0, 37, 1024, 5000)          # 5000 is clamped to N
    N = 1024
    want = oracle.pair_count(len(lens), N, 3, pats, causal, lengths=[min(x, N) for x in lens])
    assert dla.pair_count_varlen(pats, causal, lens, N, 3) == want


def test_layer_plan_check_sizes_and_errors():
    pats = ((2048, 1), (4096, 2))
    M, E = 2 * 4096, 768
    ws_f, ws_b = dla.layer_plan_check(pats, True, 0.125, 2, 4096, 12)
    attn_f, attn_b = dla.plan_check(pats, True, 0.125, 2, 4096, 12)
    # forward: attention workspace + GEMM workspace; backward holds dA, dQKV, fp32 dX besides
    assert ws_f >= attn_f and ws_b >= attn_b + M * E * (2 + 6 + 4)
    with pytest.raises(dla.DlaError) as ei:
        dla.layer_plan_check(pats, True, 0.125, 2, 4096, 0)
    assert ei.value.code == dla.DLA_E_INVALID
    with pytest.raises(dla.DlaError):
        dla.layer_plan_check(((512, 3),), True, 0.125, 1, 1024, 12)


def test_fp8_entry_points_reject_bad_arguments_before_any_launch():
    L = dla.lib()
    ok = dla.make_shape(1, 256, 2, 64, dla.DLA_BF16)
    # quantization reads bf16 only, D = 64, strides multiple of 8, B * H <= 65535
    for shape, code in ((dla.make_shape(1, 256, 2, 64, dla.DLA_F32), dla.DLA_E_UNSUPPORTED),
                        (dla.make_shape(1, 256, 2, 32, dla.DLA_BF16, (256 * 2 * 32, 2 * 32, 32)),
                         dla.DLA_E_UNSUPPORTED),
                        (dla.make_shape(1, 256, 2, 64, dla.DLA_BF16, (256 * 132, 132, 66)), dla.DLA_E_INVALID),
                        (dla.make_shape(300, 256, 300, 64, dla.DLA_BF16), dla.DLA_E_UNSUPPORTED)):
        assert L.dla_quantize_fp8(ctypes.byref(shape), 16, 16, 16, None) == code
    assert L.dla_quantize_fp8(ctypes.byref(ok), 16, 16, None, None) == dla.DLA_E_INVALID   # null scale
    assert L.dla_quantize_fp8(ctypes.byref(ok), 16, 16, 18, None) == dla.DLA_E_INVALID     # misaligned scale
    desc = dla.make_desc(((256, 1),), True, 0.125)
    f32 = dla.make_shape(1, 256, 2, 64, dla.DLA_F32)
    assert L.dla_forward_fp8kv(ctypes.byref(desc), ctypes.byref(f32), 16, 16, 16, 16, 16, 16, 16,
                               16, 1 << 20, None) == dla.DLA_E_UNSUPPORTED
    assert L.dla_forward_fp8kv(ctypes.byref(desc), ctypes.byref(ok), 16, 16, 16, None, 16, 16, 16,
                               16, 1 << 20, None) == dla.DLA_E_INVALID


@pytest.mark.parametrize("bad", ["bf16", "bnh", "strided", "shape"])
def test_backward_entry_points_reject_a_bad_lse_before_any_launch(bad):
    """The backward reads lse as a contiguous float32 [B, H, N] array: any
    other dtype, layout or shape is refused by the binding, on the host."""
    import torch
    B, N, H = 1, 256, 2
    x = torch.zeros((B, N, H, 64), dtype=torch.bfloat16)
    lse = {"bf16": torch.zeros((B, H, N), dtype=torch.bfloat16),
           "bnh": torch.zeros((B, N, H), dtype=torch.float32),
           "strided": torch.zeros((B, N, H), dtype=torch.float32).permute(0, 2, 1),
           "shape": torch.zeros((B, H, N + 1), dtype=torch.float32)}[bad]
    calls = [lambda: dla.backward(x, x, x, x, lse, x, [(64, 1)], True),
             lambda: dla.backward_varlen(x, x, x, x, lse, x, [N], [(64, 1)], True),
             lambda: dla.backward_shard(x, x, x, x, lse, x, [(64, 1)], 2 * N, 0)]
    for call in calls:
        with pytest.raises(dla.DlaError) as ei:
            call()
        assert ei.value.code == dla.DLA_E_INVALID
        assert "lse" in str(ei.value)


@pytest.mark.parametrize("env", ["1", None])
def test_planner_log_lines_only_with_dla_log(env):
    """DLA_LOG=1 makes the host planner print one line per plan to stderr;
    without it the library prints nothing."""
    code = ("from sparse_long_sequence_dilated_amd import dla\n"
            "dla.plan_check(((2048, 1), (4096, 2)), True, 0.125, 2, 8192, 3)\n")
    e = dict(os.environ)
    e.pop("DLA_LOG", None)
    if env is not None:
        e["DLA_LOG"] = env
    out = subprocess.run([os.sys.executable, "-c", code], cwd=ROOT, env=e, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    lines = [ln for ln in out.stderr.splitlines() if ln.startswith("[dla]")]
    if env is None:
        assert lines == []
    else:
        assert len(lines) == 1
        assert "B=2 N=8192 H=3 bf16 causal patterns (2048,1),(4096,2)" in lines[0]
        assert "primary=0" in lines[0] and "pairs=" in lines[0]
