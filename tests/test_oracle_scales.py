"""Pins of the oracle's per-KV-head absmax scales (CPU only).

Each check compares the oracle with something that is not the oracle:
planted maxima whose scales are exact by hand, a pure-Python brute force
(float64 quotient rounded once to float32 by struct, which equals the
correctly rounded float32 quotient because 53 >= 2*24 + 2), and the e4m3
encoder's own range (pinned in test_oracle_codec.py).
"""

import math
import struct

import numpy as np
import pytest

from oracle import e4m3
from oracle import quant as Q


def _f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


def _brute(x):
    n, h, d = x.shape
    out = []
    for hh in range(h):
        m = 0.0
        for i in range(n):
            for j in range(d):
                a = abs(float(x[i, hh, j]))
                if math.isfinite(a) and a > m:
                    m = a
        out.append(max(_f32(m / 448.0), 2.0 ** -126))
    return np.array(out, dtype=np.float32)


def test_planted_maxima_by_hand():
    x = np.zeros((5, 4, 8), np.float32)
    x[1, 0, 2] = -3.5        # 3.5 / 448 = 2^-7
    x[4, 1, 7] = 896.0       # 2.0
    x[0, 2, 0] = 448.0       # 1.0
    x[2, 3, 5] = 7.0         # 7/448 = 2^-6
    x[3, 3, 1] = -6.0        # smaller than head 3's maximum
    np.testing.assert_array_equal(Q.absmax_scales(x),
                                  np.array([2.0 ** -7, 2.0, 1.0, 2.0 ** -6], np.float32))


def test_rounded_quotient_by_hand():
    # 1/448 = 1/(7*64): float32 nearest of 1/7 is 0x3E124925, scaled by 2^-6
    x = np.ones((1, 1, 1), np.float32)
    want = np.frombuffer(struct.pack("I", 0x3E124925), np.float32)[0] * np.float32(2.0 ** -6)
    assert Q.absmax_scales(x)[0] == want


def test_non_finite_entries_are_skipped():
    x = np.ones((3, 2, 4), np.float32)
    x[0, 0, 0] = np.inf
    x[1, 0, 1] = -np.inf
    x[2, 0, 2] = np.nan
    x[2, 0, 3] = -224.0
    x[0, 1, :] = np.nan       # head 1: NaNs and ones -> absmax 1
    s = Q.absmax_scales(x)
    assert s[0] == np.float32(0.5)
    assert s[1] == np.float32(_f32(1.0 / 448.0))


def test_zero_and_empty_heads_take_the_floor():
    x = np.zeros((4, 3, 8), np.float32)
    x[2, 1, 3] = 1e-3
    s = Q.absmax_scales(x)
    assert s[0] == np.float32(2.0 ** -126) and s[2] == np.float32(2.0 ** -126)
    assert s[1] == np.float32(_f32(_f32(1e-3) / 448.0))
    e = Q.absmax_scales(np.zeros((0, 2, 8), np.float32))
    np.testing.assert_array_equal(e, np.full(2, 2.0 ** -126, np.float32))
    # a quotient below the smallest normal is raised to it
    tiny = np.full((1, 1, 2), np.float32(2.0 ** -130), np.float32)
    assert Q.absmax_scales(tiny)[0] == np.float32(2.0 ** -126)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_vs_brute_force(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((7, 3, 16)) * rng.choice([1e-3, 1.0, 50.0], size=(1, 3, 1))
         ).astype(np.float32)
    x[rng.integers(0, 7), rng.integers(0, 3), rng.integers(0, 16)] = np.nan
    np.testing.assert_array_equal(Q.absmax_scales(x), _brute(x))


def test_scale_maps_each_heads_maximum_to_the_top_code():
    # with the scale of its own head, every head's largest value encodes to
    # +-448 and no head needs saturation beyond rounding to that code
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 4, 32)) * np.array([0.01, 1.0, 30.0, 700.0])[None, :, None]
         ).astype(np.float32)
    s = Q.absmax_scales(x)
    codes = Q.quantize_rows(x, s[None, :, None])
    vals = np.abs(e4m3.decode(codes))
    for h in range(4):
        assert vals[:, h, :].max() == 448.0
        # values that end on the top code are those whose float32 quotient
        # reaches the e4m3 midpoint below 448 (432, a tie that rounds to the
        # even code 448)
        y = np.abs(np.divide(x[:, h, :], s[h], dtype=np.float32))
        assert np.all((vals[:, h, :] == 448.0) == (y >= 432.0))


def test_bf16_valued_inputs():
    import torch
    rng = np.random.default_rng(9)
    xb = torch.from_numpy(rng.standard_normal((9, 2, 8)).astype(np.float32)).bfloat16()
    x = xb.float().numpy()
    np.testing.assert_array_equal(Q.absmax_scales(x), _brute(x))
