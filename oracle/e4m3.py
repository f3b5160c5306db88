"""OCP E4M3 codec and bf16 rounding, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[BLOG] "Introduction" states that the whole FP8 attention path uses the e4m3
format; [GPUSTACK] "KV cache quantization" names E4M3 (and E5M2) as the FP8
KV formats.  Neither page gives the bit layout, so the definition used here is
the OCP OFP8 E4M3 encoding:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 encodes subnormals  m * 2**-9;
* otherwise (1 + m/8) * 2**(e - 7);
* S.1111.111 is NaN, there is no infinity; largest finite value 448 (0x7E).

Readings taken where the pages are silent (also listed in the design doc):

* rounding is round-to-nearest, ties to even mantissa;
* overflow saturates: |y| >= 448, including +-inf, encodes as +-448;
* NaN encodes as 0x7F with the input's sign bit;
* the sign of a value that rounds to zero is kept (-tiny -> 0x80).
"""

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6
_SUBNORMAL_STEP = 2.0 ** -9


def decode_code(c):
    """Value of one e4m3 code (int 0..255) as a Python float, from the format.

    Parity: pinned by the hand-listed code values and by torch's
    float8_e4m3fn view in tests/test_oracle_codec.py.
    """
    c = int(c)
    s = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * _SUBNORMAL_STEP
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def decode_table():
    """float64[256]: value of every code (NaN for 0x7F and 0xFF)."""
    return np.array([decode_code(c) for c in range(256)], dtype=np.float64)


_TABLE = decode_table()


def decode(codes):
    """Vectorised decode of a uint8 array through the 256-entry table."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(y):
    """Encode float values (fp32 or fp64 array) to e4m3 codes (uint8).

    Steps, all exact in float64 for float32 inputs:
      1. NaN -> 0x7F | sign.
      2. |y| >= 448 (this includes +-inf) -> 0x7E | sign  (saturation).
      3. |y| < 2**-6: m = round_half_even(|y| * 2**9); the code is m itself
         (m == 8 lands exactly on the smallest normal, code 0x08).
      4. otherwise e = floor(log2 |y|), m = round_half_even((|y|/2**e - 1)*8);
         a carry (m == 8) moves to exponent e + 1.  Code = (e + 7) << 3 | m.
      5. the sign bit is copied from the input (so -0 and -tiny give 0x80).

    Parity: pinned by an independent brute-force nearest-code search over all
    65,536 bf16 bit patterns and random fp32, by torch's float8_e4m3fn cast on
    inputs clamped to +-448, and by hand-listed tie cases.
    """
    y = np.asarray(y, dtype=np.float64)
    sign = np.signbit(y).astype(np.uint8) << 7
    a = np.abs(y)
    out = np.zeros(y.shape, dtype=np.uint8)

    nan = np.isnan(a)
    sat = (~nan) & (a >= E4M3_MAX)
    sub = (~nan) & (a < _MIN_NORMAL)
    nrm = ~(nan | sat | sub)

    out[nan] = 0x7F
    out[sat] = 0x7E
    out[sub] = np.rint(a[sub] / _SUBNORMAL_STEP).astype(np.uint8)

    if np.any(nrm):
        an = a[nrm]
        # frexp gives an = f * 2**k with f in [0.5, 1): floor(log2 an) = k - 1
        _, k = np.frexp(an)
        e = k.astype(np.int64) - 1
        m = np.rint((np.ldexp(an, -e) - 1.0) * 8.0).astype(np.int64)
        carry = m == 8
        m[carry] = 0
        e[carry] += 1
        out[nrm] = (((e + 7) << 3) | m).astype(np.uint8)
    return out | sign


def bf16_round(x):
    """Round float32 values to bfloat16 (nearest, ties to even); returns fp64.

    bf16 keeps 8 significant bits and float32's exponent range, subnormals
    included, so the spacing of representable values next to |x| is
    2**(max(floor(log2|x|), -126) - 7).  Rounding to that grid with ties to
    even is exact in float64.  Values whose magnitude rounds past the largest
    finite bf16 (0x7F7F) become infinities; NaN stays NaN.

    Parity: pinned against torch's float32 -> bfloat16 cast over random and
    edge bit patterns in tests/test_oracle_codec.py.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0.0)
    xf = x[fin]
    _, k = np.frexp(np.abs(xf))
    e = np.maximum(k.astype(np.int64) - 1, -126)
    ulp = np.ldexp(1.0, e - 7)
    r = np.rint(xf / ulp) * ulp
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r[np.abs(r) > bf16_max] = np.copysign(np.inf, r[np.abs(r) > bf16_max])
    out[fin] = r
    return out
