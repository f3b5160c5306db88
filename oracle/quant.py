"""Per-KV-head quantization and the paged cache write (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[BLOG] "Kernel and vLLM improvements / Per-Head Scales": the cache-write
kernel takes an array of scales, one per KV head, instead of one scalar.
[EXPLAINER] "FP8 combines value and scale": values are adjusted by the scale
before they are quantized, and the scale is applied again when attention runs.
The plainest reading of "adjusted by the scale" is a division, y = x / s, and
that is what is written here (the reading is listed in the design doc).

Cache layout (the boundary's own choice, documented in include/fa8attn.h):
  cache[num_blocks][H_kv][2][16][D], index 0 = K and 1 = V.
A token with slot id ``t`` lives in block t // 16 at row t % 16.  Negative
slot ids are padding and write nothing.
"""

import numpy as np

from . import e5m2
from .e4m3 import encode, bf16_round

BLOCK_SIZE = 16


FP8_CACHES = ("e4m3", "e5m2")


def quantize_rows(x, scale, fmt="e4m3"):
    """FP8 codes (``fmt`` e4m3 or e5m2) of fl32(fl32(x) / fl32(scale)) (scale
    broadcasts over x).

    The quotient is one IEEE float32 division (correctly rounded); its result
    is then encoded with round-to-nearest-even and saturation.  The double
    rounding (fp32 quotient, then FP8) is part of the definition.
    """
    xf = np.asarray(x, dtype=np.float32)
    sf = np.asarray(scale, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = np.divide(xf, sf, dtype=np.float32)
    if fmt == "e4m3":
        return encode(y)
    if fmt == "e5m2":
        return e5m2.encode(y)
    raise ValueError(fmt)


def bf16_bits(x):
    """uint16 bit patterns of bf16_round(x) (value -> float32 -> top 16 bits)."""
    vals = bf16_round(x).astype(np.float32)
    return (vals.view(np.uint32) >> 16).astype(np.uint16)


def new_cache(num_blocks, num_kv_heads, head_dim, cache_dtype, fill=None):
    """Host image of a paged cache: uint8 codes for 'e4m3' and 'e5m2', uint16
    bits for 'bf16'."""
    shape = (num_blocks, num_kv_heads, 2, BLOCK_SIZE, head_dim)
    dt = np.uint8 if cache_dtype in FP8_CACHES else np.uint16
    c = np.zeros(shape, dtype=dt)
    if fill is not None:
        c[...] = fill
    return c


def cache_write(cache, k, v, slot_mapping, k_scale, v_scale, cache_dtype):
    """Write K/V rows into ``cache`` in place and return it.

    k, v          float arrays [N][H_kv][D] (fp32 or bf16 values)
    slot_mapping  int array [N]; slot < 0 means "skip this row"
    k_scale/v_scale  float32 [H_kv]; ignored for the bf16 cache, whose rows
                  are the bf16 rounding of the inputs ([BLOG] "Skipping
                  layers": such layers keep BF16 and are not quantized).
    """
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    blk = slots[keep] // BLOCK_SIZE
    row = slots[keep] % BLOCK_SIZE
    kk = k[keep]
    vv = v[keep]
    if cache_dtype in FP8_CACHES:
        ks = np.asarray(k_scale, dtype=np.float32)[None, :, None]
        vs = np.asarray(v_scale, dtype=np.float32)[None, :, None]
        kc = quantize_rows(kk, ks, cache_dtype)
        vc = quantize_rows(vv, vs, cache_dtype)
    elif cache_dtype == "bf16":
        kc = bf16_bits(kk)
        vc = bf16_bits(vv)
    else:
        raise ValueError(cache_dtype)
    # cache[blk, h, 0, row, :] = kc[i, h, :]
    for h in range(k.shape[1]):
        cache[blk, h, 0, row, :] = kc[:, h, :]
        cache[blk, h, 1, row, :] = vc[:, h, :]
    return cache


def dequantize(codes, scale, cache_dtype):
    """Dequantised values in float64: scale * decode(code) for e4m3 and e5m2
    (exact: a 24-bit scale times a 4- or 3-bit significand fits in 53 bits),
    or the bf16 value for the bf16 cache."""
    if cache_dtype == "e4m3":
        from .e4m3 import decode
        return np.float64(np.float32(scale)) * decode(codes)
    if cache_dtype == "e5m2":
        return np.float64(np.float32(scale)) * e5m2.decode(codes)
    bits = np.asarray(codes, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


E4M3_MAX = 448.0
E5M2_MAX = e5m2.E5M2_MAX
SCALE_FLOOR = np.float32(2.0 ** -126)   # smallest normal float32


def absmax_scales(x, fmt_max=E4M3_MAX):
    """Per-KV-head scales from the data itself: fl32(absmax_h / fmt_max).

    [GPUSTACK] "キャリブレーション" (dynamic quantization: the value range is
    computed at run time from the data), [EXPLAINER] "default scaleのまま本番へ
    出さない" (a fixed, a dynamic or a calibrated scale), [BLOG] "Kernel and
    vLLM improvements / Per-Head Scales" (one scale per KV head).  Readings:
    the range is the largest magnitude, mapped onto the format's largest
    finite value (448 for e4m3, 57344 for e5m2), so that value encodes to the
    top code without saturating anything else.

    x    float array [N][H_kv][D] (fp32 or bf16 values)
    returns float32 [H_kv]:
        absmax_h = max |x[n][h][d]| over the finite entries (NaN and +-inf
                   are skipped; max over nothing is 0)
        scale_h  = max(fl32(absmax_h / fmt_max), 2^-126)
    The quotient is one correctly rounded float32 division; the floor keeps
    an all-zero (or empty) head's scale positive and normal.
    """
    xf = np.asarray(x, dtype=np.float32)
    if xf.ndim != 3:
        raise ValueError("x must be [N][H_kv][D]")
    a = np.abs(xf)
    a = np.where(np.isfinite(a), a, np.float32(0.0))
    if xf.shape[0] == 0:
        amax = np.zeros(xf.shape[1], dtype=np.float32)
    else:
        amax = a.max(axis=(0, 2)).astype(np.float32)
    q = np.divide(amax, np.float32(fmt_max), dtype=np.float32)
    return np.maximum(q, SCALE_FLOOR).astype(np.float32)
