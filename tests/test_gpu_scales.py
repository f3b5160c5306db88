"""GPU parity of the on-device per-KV-head absmax scales: bit-exact against
the oracle's absmax_scales, through the C ABI."""

import numpy as np
import pytest

import workloads as W
from oracle import quant as OQ
from _gpu_common import dev, log

pytestmark = pytest.mark.gpu


def _run(k, v, in_bf16):
    import torch
    import attention_fp8_quantized_amd as fa
    dt = torch.bfloat16 if in_bf16 else torch.float32
    ks, vs = fa.absmax_scales(dev(k, dt), dev(v, dt))
    torch.cuda.synchronize()
    return ks.cpu().numpy(), vs.cpu().numpy()


def _inputs(seed, shape, in_bf16, outliers=True):
    g = W.rng(7, seed, W.K)
    k = W.normal(g, shape)
    v = W.normal(W.rng(7, seed, W.V), shape)
    if outliers and shape[0] > 0:
        k = W.with_outliers(k, W.rng(7, seed, W.OUTLIERS))
    if in_bf16:
        k = W.bf16_values(k)[1]
        v = W.bf16_values(v)[1]
    return k, v


def _check(k, v, in_bf16, what):
    log(f"[absmax] {what} shape={k.shape} bf16={in_bf16}")
    gk, gv = _run(k, v, in_bf16)
    np.testing.assert_array_equal(gk.view(np.uint32), OQ.absmax_scales(k).view(np.uint32))
    np.testing.assert_array_equal(gv.view(np.uint32), OQ.absmax_scales(v).view(np.uint32))


@pytest.mark.parametrize("in_bf16", [False, True])
@pytest.mark.parametrize("shape", [
    (1, 8, 128),        # one decode row
    (8, 8, 128),        # a decode batch
    (1000, 2, 64),      # rows not a multiple of the rows per step
    (333, 64, 256),     # rows wider than one workgroup step (many columns per thread)
    (4097, 1, 256),     # head_dim 256, one KV head
    (20011, 8, 128),    # several steps per workgroup and a ragged tail
])
def test_matches_oracle_bit_exact(shape, in_bf16):
    k, v = _inputs(sum(shape) % 97, shape, in_bf16)
    _check(k, v, in_bf16, "random")


@pytest.mark.parametrize("in_bf16", [False, True])
def test_non_finite_zero_heads_and_planted_maxima(in_bf16):
    k, v = _inputs(3, (517, 4, 64), in_bf16, outliers=False)
    k[10, 0, 3] = np.inf
    k[11, 0, 4] = -np.inf
    k[12, 0, 5] = np.nan
    k[:, 1, :] = 0.0                  # all-zero head: floor scale
    k[516, 2, 63] = -896.0            # last row, last channel: scale 2.0
    v[:, 3, :] = np.nan               # head of NaNs only: floor scale
    v[0, 0, 0] = 448.0                # first element: scale 1.0
    _check(k, v, in_bf16, "planted")
    gk, gv = _run(k, v, in_bf16)
    assert gk[2] == np.float32(2.0) and gv[0] == np.float32(1.0)
    assert gk[1] == np.float32(2.0 ** -126) and gv[3] == np.float32(2.0 ** -126)


@pytest.mark.parametrize("in_bf16", [False, True])
def test_e5m2_scales(in_bf16):
    import torch
    import attention_fp8_quantized_amd as fa
    k, v = _inputs(6, (2000, 8, 128), in_bf16)
    dt = torch.bfloat16 if in_bf16 else torch.float32
    log(f"[absmax] e5m2 bf16={in_bf16}")
    ks, vs = fa.absmax_scales(dev(k, dt), dev(v, dt), cache_dtype="e5m2")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ks.cpu().numpy().view(np.uint32),
                                  OQ.absmax_scales(k, OQ.E5M2_MAX).view(np.uint32))
    np.testing.assert_array_equal(vs.cpu().numpy().view(np.uint32),
                                  OQ.absmax_scales(v, OQ.E5M2_MAX).view(np.uint32))


def test_empty_input_writes_the_floor():
    import torch
    import attention_fp8_quantized_amd as fa
    k = torch.zeros((0, 3, 128), dtype=torch.float32, device="cuda")
    ks = torch.full((3,), 5.0, device="cuda")
    vs = torch.full((3,), 5.0, device="cuda")
    fa.absmax_scales(k, k.clone(), ks, vs)
    torch.cuda.synchronize()
    assert np.all(ks.cpu().numpy() == np.float32(2.0 ** -126))
    assert np.all(vs.cpu().numpy() == np.float32(2.0 ** -126))


def test_repeated_calls_do_not_accumulate():
    # the scale arrays are both the accumulator and the result: a second call
    # with smaller data must not keep the first call's maximum
    k, v = _inputs(5, (300, 8, 128), False)
    _check(k, v, False, "first")
    _check(k * np.float32(0.25), v * np.float32(0.5), False, "second, smaller")


def test_full_size_128k_layer():
    """Llama-3.1-8B-shaped layer at 128k tokens (the bulk fill of the
    longest decode context), fp32 rows: 512 MiB each for k and v."""
    import torch
    import attention_fp8_quantized_amd as fa
    n, h, d = 131072, 8, 128
    g = torch.Generator(device="cuda").manual_seed(11)
    k = torch.randn((n, h, d), device="cuda", generator=g)
    v = torch.randn((n, h, d), device="cuda", generator=g)
    k[:, 3, 17] *= 20.0
    log(f"[absmax] full size {n}x{h}x{d} fp32")
    ks, vs = fa.absmax_scales(k, v)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ks.cpu().numpy().view(np.uint32),
                                  OQ.absmax_scales(k.cpu().numpy()).view(np.uint32))
    np.testing.assert_array_equal(vs.cpu().numpy().view(np.uint32),
                                  OQ.absmax_scales(v.cpu().numpy()).view(np.uint32))
