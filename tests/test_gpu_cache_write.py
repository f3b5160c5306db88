"""GPU cache write vs the oracle: bit-exact cache bytes.

e4m3 / e5m2 cache: code = fp8(fl32(x / scale[h])) with round-to-nearest-even
and saturation; bf16 cache: bf16 rounding of x.  Checked exhaustively over every
bf16 bit pattern at four scales, on random fp32 at several magnitudes, on an
edge set (ties, saturation, inf, NaN, fp32 subnormals, signed zeros), through
both input dtypes, and with a sentinel-filled cache to prove that only the
mapped slots change.
"""

import numpy as np
import pytest

import workloads as W
from oracle import quant as OQ

from _gpu_common import dev, log

pytestmark = pytest.mark.gpu


def _gpu_write(k, v, slots, ks, vs, nblocks, Hkv, D, cd, in_bf16=False, fill=None):
    import torch
    import attention_fp8_quantized_amd as fa
    slots = np.asarray(slots, np.int64)
    # host-side bounds check before anything is launched
    assert slots.max() < nblocks * 16 and len(np.unique(slots[slots >= 0])) == (slots >= 0).sum()
    assert k.shape == v.shape == (len(slots), Hkv, D)
    cache = fa.new_cache(nblocks, Hkv, D, cd)
    if fill is not None:
        cache.view(torch.uint8).fill_(fill)
    kt, vt = dev(k), dev(v)
    if in_bf16:
        def to_bf16(a):
            bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
            if np.all((bits & 0xFFFF) == 0):
                # exact bf16 patterns: keep every bit (torch's cast would
                # replace NaN payloads and signs by its canonical NaN)
                hi = (bits >> 16).astype(np.uint16).view(np.int16)
                return torch.from_numpy(hi).cuda().view(torch.bfloat16)
            return dev(a).to(torch.bfloat16)
        kt, vt = to_bf16(k), to_bf16(v)
    fa.cache_write(kt, vt, dev(np.asarray(slots, np.int64)), dev(ks), dev(vs), cache)
    torch.cuda.synchronize()
    out = cache.cpu()
    if cd == "bf16":
        return out.view(torch.int16).numpy().view(np.uint16)
    return out.view(torch.uint8).numpy()


def _oracle_write(k, v, slots, ks, vs, nblocks, Hkv, D, cd, fill=None):
    c = OQ.new_cache(nblocks, Hkv, D, cd, fill=fill)
    return OQ.cache_write(c, k, v, slots, ks, vs, cd)


def _all_bf16_as_f32():
    return (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("cd", ["e4m3", "e5m2"])
@pytest.mark.parametrize("scale", [1.0, 0.0123, 2.0 ** -5, 7.0])
def test_exhaustive_bf16_patterns(scale, cd):
    # at s = 7 the correctly rounded x / s and x * fl32(1 / s) encode 60 of
    # the bf16 patterns differently in each format (tests/golden/
    # quantize_division.txt works three of them by hand), so the K rows
    # compare the division itself
    Hkv, D = 2, 128
    x = _all_bf16_as_f32().reshape(-1, Hkv, D)             # 256 tokens
    v = -x[::-1].copy()
    N = x.shape[0]
    slots = np.random.default_rng(1).permutation(N + 32)[:N]
    nblocks = (N + 32 + 15) // 16
    ks = np.full(Hkv, scale, np.float32)
    vs = np.array([scale, scale * 3], np.float32)
    log(f"cache_write exhaustive bf16 patterns scale={scale} cache={cd}")
    want = _oracle_write(x, v, slots, ks, vs, nblocks, Hkv, D, cd, fill=0xA5)
    got = _gpu_write(x, v, slots, ks, vs, nblocks, Hkv, D, cd, fill=0xA5)
    assert np.array_equal(got, want)
    # same values arriving as bf16 tensors (exact: they are bf16 patterns)
    got_b = _gpu_write(x, v, slots, ks, vs, nblocks, Hkv, D, cd, in_bf16=True, fill=0xA5)
    assert np.array_equal(got_b, want)


def _edge_values():
    f = np.float32
    ulp448 = np.nextafter(f(448), f(1e9))
    vals = [448, -448, 464, -464, 480, -480, ulp448, -ulp448, 2 ** -10, -2 ** -10,
            3 * 2 ** -11, 2 ** -6, np.nextafter(f(2 ** -6), f(0)), np.nextafter(f(2 ** -6), f(1)),
            1e-45, -1e-45, 1e-40, 0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, 1.0625, 1.1875,
            3e38, -3e38, 432.0, 424.0,
            # e5m2: saturation, ties, subnormal and smallest-normal edges
            57344, -57344, 61440, -61440, 57345, np.nextafter(f(61440), f(0)), 1.125, 1.375,
            1.875, 53248.0, 2 ** -17, 3 * 2 ** -17, 7 * 2 ** -17, 2 ** -14,
            np.nextafter(f(2 ** -14), f(0))]
    return np.array(vals, dtype=np.float32)


@pytest.mark.parametrize("cd", ["e4m3", "e5m2"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_random_and_edges(D, cd):
    g = np.random.default_rng(D)
    Hkv = 4
    N = 300
    parts = [g.standard_normal(N * Hkv * D // 4).astype(np.float32) * m for m in (1, 20, 1000)]
    edges = np.resize(_edge_values(), N * Hkv * D - sum(p.size for p in parts))
    x = np.concatenate(parts + [edges]).astype(np.float32)
    g.shuffle(x)
    k = x.reshape(N, Hkv, D)
    v = np.roll(x, 7).reshape(N, Hkv, D)
    ks = g.uniform(0.001, 3.0, Hkv).astype(np.float32)
    vs = g.uniform(0.001, 3.0, Hkv).astype(np.float32)
    slots = g.permutation(N * 2)[:N]
    nb = (N * 2 + 15) // 16
    log(f"cache_write random+edges D={D} cache={cd}")
    want = _oracle_write(k, v, slots, ks, vs, nb, Hkv, D, cd, fill=0xA5)
    got = _gpu_write(k, v, slots, ks, vs, nb, Hkv, D, cd, fill=0xA5)
    assert np.array_equal(got, want)


def test_negative_slots_skip_and_sentinel():
    g = np.random.default_rng(3)
    Hkv, D, N = 2, 64, 40
    k = g.standard_normal((N, Hkv, D)).astype(np.float32)
    v = g.standard_normal((N, Hkv, D)).astype(np.float32)
    slots = np.arange(N, dtype=np.int64) * 3
    slots[::4] = -1
    nb = (3 * N + 15) // 16
    one = np.ones(Hkv, np.float32)
    log("cache_write negative slots + sentinel")
    want = _oracle_write(k, v, slots, one, one, nb, Hkv, D, "e4m3", fill=0xA5)
    got = _gpu_write(k, v, slots, one, one, nb, Hkv, D, "e4m3", fill=0xA5)
    assert np.array_equal(got, want)
    assert np.sum(got != 0xA5) <= (slots >= 0).sum() * Hkv * D * 2


@pytest.mark.parametrize("in_bf16", [False, True])
def test_bf16_cache(in_bf16):
    g = np.random.default_rng(4)
    Hkv, D, N = 2, 128, 200
    x = np.concatenate([_all_bf16_as_f32()[:N * Hkv * D // 2],
                        g.standard_normal(N * Hkv * D // 2).astype(np.float32)])
    if not in_bf16:
        x[1::7] += np.float32(1e-3)       # values that really need rounding
    k = x.reshape(N, Hkv, D)
    v = -k
    slots = g.permutation(N + 16)[:N]
    nb = (N + 16 + 15) // 16
    one = np.ones(Hkv, np.float32)
    log(f"cache_write bf16 cache in_bf16={in_bf16}")
    want = _oracle_write(k, v, slots, one, one, nb, Hkv, D, "bf16")
    got = _gpu_write(k, v, slots, one, one, nb, Hkv, D, "bf16", in_bf16=in_bf16, fill=0)
    nan_w = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
    nan_g = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    assert np.array_equal(nan_w, nan_g)
    assert np.array_equal(got[~nan_w], want[~nan_w])


@pytest.mark.parametrize("cd", ["e4m3", "e5m2"])
@pytest.mark.parametrize("N", [1, 8])
def test_decode_step_sized_write(N, cd):
    # one new token per sequence, Llama-shaped heads, per-head absmax scales
    Hkv, D = 8, 128
    g = W.rng(2, 0, W.K)
    k = W.normal(g, (N, Hkv, D))
    v = W.normal(g, (N, Hkv, D))
    ks = np.random.default_rng(5).uniform(0.002, 0.05, Hkv).astype(np.float32)
    vs = np.random.default_rng(6).uniform(0.002, 0.05, Hkv).astype(np.float32)
    slots = np.arange(N, dtype=np.int64) * 16 + 5
    nb = N
    log(f"cache_write decode-step N={N} cache={cd}")
    want = _oracle_write(k, v, slots, ks, vs, nb, Hkv, D, cd, fill=0xA5)
    got = _gpu_write(k, v, slots, ks, vs, nb, Hkv, D, cd, fill=0xA5)
    assert np.array_equal(got, want)
