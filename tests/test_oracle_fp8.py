"""Pins of the 8-bit key/value oracle (CPU only).

  * the E4M3 decode table against torch's float8_e4m3fn for all 256 codes;
  * the encoder against torch's round-to-nearest-even cast to float8_e4m3fn,
    on every representable value, every midpoint between neighbours (the
    ties), values just off the midpoints, subnormals and random values;
  * per-head quantization: the largest magnitude of a head maps to the code
    of +-448, the dequantized values lie within half a step of the inputs,
    and an all-zero head gets codes 0 and scale 1.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_long_sequence_dilated_amd import inputs


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_matches_torch_e4m3fn():
    mine = oracle.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(mine[~np.isnan(mine)], ref[~np.isnan(ref)])
    assert np.nanmax(mine) == 448.0 and np.nanmin(mine) == -448.0


def test_encode_matches_torch_rounding():
    t = oracle.e4m3_decode_table()
    pos = np.unique(t[(t >= 0) & ~np.isnan(t)])
    mids = (pos[1:] + pos[:-1]) / 2
    g = np.random.Generator(np.random.PCG64(11))
    rnd = np.clip(g.standard_normal(20000) * 40, -448, 448)
    sub = g.uniform(-2.0 ** -6, 2.0 ** -6, 5000)
    vals = np.concatenate([pos, -pos, mids, -mids, mids * (1 + 2 ** -20), mids * (1 - 2 ** -20),
                           rnd, sub, [0.0, -0.0, 1e-30, -1e-30, 448.0, -448.0]]).astype(np.float32)
    vals = vals[np.abs(vals) <= 448]
    assert np.array_equal(oracle.e4m3_encode(vals), _torch_codes(vals))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([449.0]))


def test_quantize_per_head_properties():
    x, = inputs.draw((2, 300, 3, 64), 21, 1, "bf16")
    x[1, :, 2] *= 1e-3                        # a head of small values: more subnormal codes
    x[0, :, 1] = 0.0                          # an all-zero head
    codes, scale = oracle.quantize_per_head(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32 and scale.shape == (2, 3)
    assert np.all(codes[0, :, 1] == 0) and scale[0, 1] == 1.0
    deq = oracle.dequantize_per_head(codes, scale)
    for b in range(2):
        for h in range(3):
            xs = x[b, :, h].astype(np.float64)
            if not np.any(xs):
                continue
            amax = np.abs(xs).max()
            assert scale[b, h] == np.float32(np.float32(amax) / np.float32(448))
            i = np.unravel_index(np.argmax(np.abs(xs)), xs.shape)
            assert codes[b, :, h][i] & 0x7F == 0x7E  # +-448
            # half a step: 2^-4 relative for normal codes, 2^-10 * scale for subnormals
            s = np.float64(scale[b, h])
            bound = np.maximum(np.abs(xs) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-5)
            assert np.all(np.abs(deq[b, :, h] - xs) <= bound)
