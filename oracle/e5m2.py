"""OCP E5M2 codec, written from the format definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[GPUSTACK] "KV キャッシュの量子化" names E5M2 next to E4M3 as the FP8 formats
a KV cache may use.  The page gives no bit layout; the definition used here
is the OCP OFP8 E5M2 encoding:

* 1 sign bit, 5 exponent bits (bias 15), 2 mantissa bits;
* exponent field 0 encodes subnormals  m * 2**-16;
* exponent fields 1..30 encode (1 + m/4) * 2**(e - 15);
* exponent field 31 is +-inf (m = 0) or NaN (m != 0); largest finite value
  57344 (0x7B).

Readings taken where the pages are silent (the same rules as the e4m3
cache, so both caches share one contract):

* rounding is round-to-nearest, ties to even mantissa;
* overflow saturates: |y| >= 57344, including +-inf, encodes as +-57344, so
  the cache never holds an infinity;
* NaN encodes as 0x7F (S.11111.11) with the input's sign bit;
* the sign of a value that rounds to zero is kept (-tiny -> 0x80).
"""

import numpy as np

E5M2_MAX = 57344.0
_MIN_NORMAL = 2.0 ** -14
_SUBNORMAL_STEP = 2.0 ** -16


def decode_code(c):
    """Value of one e5m2 code (int 0..255) as a Python float, from the format.

    Parity: pinned by hand-listed code values and by torch's float8_e5m2
    view in tests/test_oracle_e5m2.py.
    """
    c = int(c)
    s = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 2) & 0x1F
    m = c & 0x3
    if e == 0x1F:
        return s * float("inf") if m == 0 else float("nan")
    if e == 0:
        return s * m * _SUBNORMAL_STEP
    return s * (1.0 + m / 4.0) * 2.0 ** (e - 15)


def decode_table():
    """float64[256]: value of every code (+-inf for 0x7C/0xFC, NaN for the
    other exponent-31 codes)."""
    return np.array([decode_code(c) for c in range(256)], dtype=np.float64)


_TABLE = decode_table()


def decode(codes):
    """Vectorised decode of a uint8 array through the 256-entry table."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(y):
    """Encode float values (fp32 or fp64 array) to e5m2 codes (uint8).

    Steps, all exact in float64 for float32 inputs:
      1. NaN -> 0x7F | sign.
      2. |y| >= 57344 (this includes +-inf) -> 0x7B | sign  (saturation).
      3. |y| < 2**-14: m = round_half_even(|y| * 2**16); the code is m itself
         (m == 4 lands exactly on the smallest normal, code 0x04).
      4. otherwise e = floor(log2 |y|), m = round_half_even((|y|/2**e - 1)*4);
         a carry (m == 4) moves to exponent e + 1.  Code = (e + 15) << 2 | m
         (a carry out of 2**15 cannot happen below 57344: 1.75*2**15 is the
         top of that binade and values above it saturated in step 2).
      5. the sign bit is copied from the input (so -0 and -tiny give 0x80).

    Parity: pinned by an independent brute-force nearest-code search over all
    65,536 bf16 bit patterns and random fp32, by torch's float8_e5m2 cast on
    inputs clamped to +-57344, and by hand-listed tie cases.
    """
    y = np.asarray(y, dtype=np.float64)
    sign = np.signbit(y).astype(np.uint8) << 7
    a = np.abs(y)
    out = np.zeros(y.shape, dtype=np.uint8)

    nan = np.isnan(y)
    sat = ~nan & (a >= E5M2_MAX)
    sub = ~nan & ~sat & (a < _MIN_NORMAL)
    nrm = ~nan & ~sat & ~sub

    out[nan] = 0x7F
    out[sat] = 0x7B
    out[sub] = np.rint(a[sub] / _SUBNORMAL_STEP).astype(np.uint8)  # rint: ties to even

    an = a[nrm]
    e = np.floor(np.log2(an)).astype(np.int64)
    # floor(log2) can be off by one next to a power of two; fix it exactly
    e = np.where(np.ldexp(1.0, e) > an, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= an, e + 1, e)
    frac = an / np.ldexp(1.0, e) - 1.0                      # in [0, 1), exact
    m = np.rint(frac * 4.0).astype(np.int64)                 # ties to even
    carry = m == 4
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    out[nrm] = (((e + 15) << 2) | m).astype(np.uint8)

    return out | sign
