"""Pins of the oracle's e5m2 codec (CPU only).

Each check compares the oracle with something that is not the oracle:
hand-derived values from the OCP E5M2 definition (tests/golden), torch's own
float8_e5m2 dtype, and an independent brute-force nearest-code search.
"""

import math
import os

import numpy as np
import torch

from oracle import e5m2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name, code_first):
    """Rows of (code, expression) or (expression, code); an expression may
    hold spaces, the code is one token."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split(None, 1) if code_first else line.rsplit(None, 1))
    return rows


def _same(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_code_values_match_hand_table():
    rows = _read_golden("e5m2_codes.txt", True)
    assert len(rows) >= 20
    for code, expr in rows:
        want = float(eval(expr))  # noqa: S307 - fixture of literals
        assert _same(e5m2.decode_code(int(code, 16)), want), (code, expr)


def test_all_codes_match_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    got = e5m2.decode_table()
    for c in range(256):
        assert _same(float(got[c]), float(ref[c])), hex(c)


def test_round_trip_all_finite_codes():
    vals = e5m2.decode_table()
    fin = np.isfinite(vals)
    codes = np.arange(256, dtype=np.uint8)[fin]
    assert np.array_equal(e5m2.encode(vals[fin]), codes)


def test_rounding_ties_and_saturation_by_hand():
    rows = _read_golden("e5m2_rounding.txt", False)
    assert len(rows) >= 15
    for expr, code in rows:
        x = np.array([float(eval(expr))], dtype=np.float32)  # noqa: S307
        assert int(e5m2.encode(x)[0]) == int(code, 16), (expr, code)


def test_nan_keeps_sign():
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    x[1] = -np.abs(x[1])
    assert e5m2.encode(x).tolist() == [0x7F, 0xFF]


def _brute_force_encode(y):
    """Nearest finite code by exhaustive search, ties to even mantissa bit,
    saturating at +-57344, sign bit copied from the input.  Written without
    any of the oracle's exponent/mantissa arithmetic."""
    y = np.asarray(y, dtype=np.float64)
    pos_codes = np.arange(0x7C, dtype=np.int64)                    # 0x00..0x7B
    pos_vals = np.array([e5m2.decode_code(c) for c in pos_codes])
    assert np.all(np.diff(pos_vals) > 0)
    sign = np.signbit(y).astype(np.uint8) << 7
    a = np.abs(y)
    isnan = np.isnan(a)
    a_fin = np.where(isnan, 0.0, np.minimum(a, 57344.0))
    d = np.abs(a_fin[:, None] - pos_vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = (pos_codes & 1) == 0
    pick_even = cand & even[None, :]
    idx = np.where(pick_even.any(axis=1), pick_even.argmax(axis=1), cand.argmax(axis=1))
    out = pos_codes[idx].astype(np.uint8)
    out[isnan] = 0x7F
    return out | sign


def _all_bf16_patterns_as_f32():
    return (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)


def test_exhaustive_bf16_patterns_vs_brute_force():
    x = _all_bf16_patterns_as_f32()
    for s in (1.0, 0.0123, 2.0 ** 10):
        with np.errstate(all="ignore"):
            y = np.divide(x, np.float32(s), dtype=np.float32)
        for chunk in np.array_split(np.arange(y.size), 16):
            assert np.array_equal(e5m2.encode(y[chunk]), _brute_force_encode(y[chunk])), s


def test_random_fp32_vs_brute_force():
    g = np.random.default_rng(17)
    for mag in (1.0, 1e-4, 3e3, 4e4):
        y = (g.standard_normal(20000) * mag).astype(np.float32)
        assert np.array_equal(e5m2.encode(y), _brute_force_encode(y)), mag


def test_matches_torch_cast_after_clamp():
    g = np.random.default_rng(19)
    x = np.concatenate([
        _all_bf16_patterns_as_f32(),
        (g.standard_normal(200000) * 3000).astype(np.float32),
        g.uniform(-2.0 ** -14, 2.0 ** -14, 50000).astype(np.float32),
    ])
    x = x[~np.isnan(x)]
    clamped = np.clip(x, -57344.0, 57344.0).astype(np.float32)
    ref = torch.from_numpy(clamped).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(ref, e5m2.encode(x))


def test_encode_is_monotone():
    x = np.sort(np.random.default_rng(23).standard_normal(100000).astype(np.float32) * 2e4)
    v = e5m2.decode(e5m2.encode(x))
    assert np.all(np.diff(v) >= 0)
