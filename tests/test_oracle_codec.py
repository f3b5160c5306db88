"""Pins of the oracle's e4m3 codec and bf16 rounding (CPU only).

Each check compares the oracle with something that is not the oracle:
hand-derived values from the OCP E4M3 definition (tests/golden), an
independent brute-force nearest-code search, and torch's own float8_e4m3fn
and bfloat16 casts.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_code_values_match_hand_table():
    rows = _read_golden("e4m3_codes.txt")
    assert len(rows) >= 20
    for code_s, *expr in rows:
        code = int(code_s, 16)
        want = eval(" ".join(expr), {"nan": float("nan")})
        got = e4m3.decode_code(code)
        if math.isnan(want):
            assert math.isnan(got), hex(code)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), hex(code)


def test_all_codes_match_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3.decode_table()
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(got))
    assert set(np.nonzero(nan_ref)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan_ref], got[~nan_ref])
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(got[~nan_ref]))


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3.encode(e4m3.decode(codes)), codes)


def test_rounding_ties_and_saturation_by_hand():
    for row in _read_golden("e4m3_rounding.txt"):
        expr, code_s = " ".join(row[:-1]), row[-1]
        x = np.float32(eval(expr, {"float": float}))
        got = int(e4m3.encode(np.array([x], dtype=np.float32))[0])
        assert got == int(code_s, 16), (expr, hex(got))


def test_nan_keeps_sign():
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    assert e4m3.encode(x).tolist() == [0x7F, 0xFF]


# --- independent brute-force encoder ------------------------------------------

def _brute_force_encode(y):
    """Nearest finite code by exhaustive search, ties to even mantissa bit,
    saturating at +-448, sign bit copied from the input.  Written without
    any of the oracle's exponent/mantissa arithmetic."""
    y = np.asarray(y, dtype=np.float64)
    pos_codes = np.array([c for c in range(0x7F)], dtype=np.int64)       # 0x00..0x7E
    pos_vals = np.array([e4m3.decode_code(c) for c in pos_codes])       # ascending
    assert np.all(np.diff(pos_vals) > 0)
    out = np.zeros(y.shape, dtype=np.uint8)
    sign = (np.signbit(y).astype(np.uint8) << 7)
    a = np.abs(y)
    isnan = np.isnan(a)
    a_fin = np.where(isnan, 0.0, np.minimum(a, 448.0))
    d = np.abs(a_fin[:, None] - pos_vals[None, :])                       # [n][127]
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes prefer the even mantissa (code & 1 == 0)
    even = (pos_codes & 1) == 0
    pick_even = cand & even[None, :]
    has_even = pick_even.any(axis=1)
    idx = np.where(has_even, pick_even.argmax(axis=1), cand.argmax(axis=1))
    out[:] = pos_codes[idx]
    out[isnan] = 0x7F
    return out | sign


def _all_bf16_patterns_as_f32():
    bits = np.arange(65536, dtype=np.uint32) << 16
    return bits.view(np.float32)


def test_exhaustive_bf16_patterns_vs_brute_force():
    x = _all_bf16_patterns_as_f32()
    for s in (1.0, 0.0123, 2.0 ** -5):
        with np.errstate(all="ignore"):
            y = np.divide(x, np.float32(s), dtype=np.float32)
        for chunk in np.array_split(np.arange(y.size), 16):
            assert np.array_equal(e4m3.encode(y[chunk]), _brute_force_encode(y[chunk])), s


def test_random_fp32_vs_brute_force():
    g = np.random.default_rng(7)
    for mag in (1.0, 20.0, 1000.0, 1e-3):
        y = (g.standard_normal(20000) * mag).astype(np.float32)
        assert np.array_equal(e4m3.encode(y), _brute_force_encode(y)), mag


def test_matches_torch_cast_after_clamp():
    g = np.random.default_rng(11)
    x = np.concatenate([
        _all_bf16_patterns_as_f32(),
        (g.standard_normal(200000) * 50).astype(np.float32),
        g.uniform(-2.0 ** -6, 2.0 ** -6, 50000).astype(np.float32),
    ])
    x = x[~np.isnan(x)]
    clamped = np.clip(x, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3.encode(x)
    assert np.array_equal(ref, got)


def test_encode_is_monotone():
    x = np.sort(np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 300)
    v = e4m3.decode(e4m3.encode(x))
    assert np.all(np.diff(v) >= 0)


# --- bf16 rounding -------------------------------------------------------------

def test_bf16_round_matches_torch():
    g = np.random.default_rng(5)
    bits = np.concatenate([
        g.integers(0, 2 ** 32, 500000, dtype=np.uint64).astype(np.uint32),
        np.arange(0, 1 << 20, 7, dtype=np.uint32),                   # fp32 subnormals
        (np.uint32(0x7F7F0000) + np.arange(0, 1 << 16, dtype=np.uint32)),  # near overflow
        np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x3F808000,
                  0x3F818000, 0x3F7FFFFF], dtype=np.uint32),
    ])
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = e4m3.bf16_round(x)
    assert np.array_equal(np.isinf(ref), np.isinf(got))
    assert np.array_equal(ref, got)
    assert np.array_equal(np.signbit(ref), np.signbit(got))


@pytest.mark.parametrize("x,want", [(1.0 + 2 ** -8, 1.0), (1.0 + 3 * 2 ** -8, 1.0 + 2 ** -6),
                                    (1.0 + 2 ** -8 + 2 ** -20, 1.0 + 2 ** -7)])
def test_bf16_ties_by_hand(x, want):
    # bf16 keeps 7 stored mantissa bits: the grid next to 1 is 2**-7
    assert e4m3.bf16_round(np.array([x], dtype=np.float32))[0] == want
