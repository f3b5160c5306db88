"""The allocation-free decode entry point (fa8_decode_attention_noalloc)
against the workspace entry point (fa8_decode_attention) it mirrors.

Both run the same kernels; the no-alloc call keeps its partials and arrival
counters in the library's fixed per-GPU scratch.  Its output must equal the
workspace call's bit for bit (and pass the oracle gate) on consecutive calls
whose scratch layouts differ: a large call, then a smaller one, then one
with a two-level split merge, then the first again.  (The refusal of a
layout beyond the scratch is a host check, tested without a GPU in
test_abi.py.)
"""

import numpy as np
import pytest

from _gpu_common import DecodeCase, assert_gate, log

pytestmark = pytest.mark.gpu


def _both(case, num_splits=0):
    import torch
    import attention_fp8_quantized_amd as fa
    ref = case.run_gpu(num_splits=num_splits)
    out = torch.full((case.B, case.Hq, case.D), float("nan"), device="cuda")
    fa.decode_attention_noalloc(case.q_dev, case.cache, case.bt_dev, case.lens_dev,
                                case.ks_dev, case.vs_dev, float(case.sm),
                                int(case.lens.max()) if case.B else 0, out,
                                window=case.window, num_splits=num_splits)
    torch.cuda.synchronize()
    return ref, out.cpu().numpy()


def _check(case, what, num_splits=0):
    log(f"decode_noalloc {what}")
    ref, got = _both(case, num_splits)
    assert np.array_equal(ref, got), f"{what}: differs from the workspace entry point"
    oref, qheads = case.oracle()
    assert_gate(got[:, qheads], oref, f"noalloc {what}")


def test_noalloc_equals_workspace_entry_point_on_consecutive_calls():
    big = DecodeCase(4, 32, 8, 128, [5000, 3333, 17, 0], "e4m3", seed=80, outliers=True,
                     oracle_heads=[0, 7])
    small = DecodeCase(1, 8, 2, 64, [300], "e4m3", seed=81)
    _check(big, "llama-shaped batch 4")
    _check(small, "hd64 batch 1 (smaller layout)")
    # 100 splits: arrivals counted per split group, the merge shared by the
    # group finishers (the set and merger counters)
    two = DecodeCase(2, 16, 2, 256, [4000, 1777], "e5m2", seed=82)
    _check(two, "hd256 sliced merge", num_splits=100)
    _check(small, "hd64 again after the two-level layout")
    _check(big, "llama-shaped again")


def test_noalloc_bf16_cache_and_window():
    c = DecodeCase(3, 16, 2, 128, [1000, 129, 5], "bf16", seed=83, window=128)
    _check(c, "bf16 window 128")
    c2 = DecodeCase(2, 16, 2, 128, [700, 40], "e4m3", seed=84, window=100, fill=0xFF,
                    window_only=True)
    _check(c2, "e4m3 window 100, NaN outside the window")
