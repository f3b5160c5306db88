"""GPU FP8 prefill vs the tile-mirrored fp64 oracle.

The oracle quantises P exactly where the method does (per 128-key tile at
absolute aligned positions, against the running row maximum after that tile)
and keeps the softmax denominator unquantised.  Gate: max |gpu - oracle| <=
2e-3 and relative L2 <= 1e-3 over the compared rows, the same bound from 200
to 131072 keys.  The unquantised-P reference (prefill_exact) is reported.
Large cases compare seeded sampled rows (always including the last 16).
"""

import numpy as np
import pytest

from _gpu_common import PrefillCase, assert_gate, log, metrics

pytestmark = pytest.mark.gpu


def _sample_rows(T, n, seed):
    g = np.random.default_rng(seed)
    tail = np.arange(max(0, T - 16), T)
    rest = g.choice(max(T - 16, 1), size=min(n - len(tail), max(T - 16, 0)), replace=False)
    return np.unique(np.concatenate([rest, tail])).astype(np.int64)


@pytest.mark.parametrize("cd", ["e4m3", "e5m2"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_single_chunk_all_rows(D, cd):
    c = PrefillCase([200], [200], 4, 2, D, seed=D, cache_dtype=cd)
    log(f"prefill D={D} T=200 cache={cd}")
    got = c.run_gpu()
    ref, slack = c.oracle()
    assert_gate(got, ref, f"D={D} T=200 {cd} mirror", slack=slack)
    ma, rl = metrics(got, c.oracle(exact=True))
    log(f"  vs unquantised-P reference: max_abs={ma:.3e} rel_l2={rl:.3e}")


@pytest.mark.parametrize("cd", ["e4m3", "e5m2"])
@pytest.mark.parametrize("window", [0, 100])
def test_chunked_ragged_batch_gqa(window, cd):
    # three sequences: fresh (P=0), continued (P=300), short tail chunk
    c = PrefillCase([130, 100, 17], [130, 400, 260], 8, 2, 128, seed=7, window=window,
                    cache_dtype=cd)
    log(f"prefill ragged window={window} cache={cd}")
    ref, slack = c.oracle()
    assert_gate(c.run_gpu(), ref, f"ragged batch window={window} {cd}", slack=slack)


@pytest.mark.parametrize("cd", ["e4m3", "e5m2"])
def test_stale_nan_rows_past_sequence_end(cd):
    # pages are pre-filled with NaN codes (0xFF in both FP8 formats); the rows
    # past each sequence end keep them and must not reach the output
    c = PrefillCase([130, 75], [130, 333], 4, 2, 128, seed=8, fill=0xFF, cache_dtype=cd)
    log(f"prefill stale NaN rows cache={cd}")
    got = c.run_gpu()
    assert np.all(np.isfinite(got))
    ref, slack = c.oracle()
    assert_gate(got, ref, "stale NaN rows", slack=slack)


def test_uniform_scores_mean_of_visible_v():
    from oracle import e4m3
    c = PrefillCase([70], [150], 2, 1, 64, seed=9, q_zero=True, q_scale=1.0)
    got = c.run_gpu()
    P = 150 - 70
    for i in [0, 5, 69]:
        pos = P + i
        codes = np.stack([np.frombuffer(e4m3.encode(c.v[t, 0] / c.vs[0]).tobytes(), np.uint8)
                          for t in range(pos + 1)])
        mean = e4m3.decode(codes).mean(axis=0) * np.float64(c.vs[0])
        for hq in range(2):
            ma, rl = metrics(got[i, hq], mean)
            assert ma < 1e-5 and rl < 1e-5, (i, hq, ma, rl)


@pytest.mark.parametrize("accum_mode", [1, 0, 2, 8])
def test_hd256_1k_all_rows(accum_mode):
    # 8 q / 1 KV head, head_dim 256, absmax scales (Q per tensor, K/V per head)
    c = PrefillCase([1024], [1024], 8, 1, 256, seed=11)
    log(f"prefill hd256 T=1024 accum_mode={accum_mode}")
    ref, slack = c.oracle()
    assert_gate(c.run_gpu(accum_mode), ref, f"hd256 T=1024 accum={accum_mode}", slack=slack)


@pytest.mark.parametrize("T", [8192, 32768])
def test_hd256_long_chunk_sampled(T):
    c = PrefillCase([T], [T], 8, 1, 256, seed=12)
    rows = _sample_rows(T, 48, seed=T)
    log(f"prefill hd256 T={T} (sampled {len(rows)} rows)")
    got = c.run_gpu()
    ref, slack = c.oracle(rows=rows)
    assert_gate(got[rows], ref, f"hd256 T={T} sampled", slack=slack)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("accum_mode", [2, 3, 16])
def test_flush_every_n_tiles(D, accum_mode):
    # flush periods that do and do not divide the tile counts of a ragged
    # chunked batch (one row sees 1 tile, another 8)
    c = PrefillCase([130, 100, 17], [130, 1000, 260], 8, 2, D, seed=15)
    log(f"prefill flush every {accum_mode} tiles D={D}")
    ref, slack = c.oracle()
    assert_gate(c.run_gpu(accum_mode), ref, f"flush/{accum_mode} D={D}", slack=slack)


def test_accumulation_modes_at_32k():
    """Every accumulation mode on the 32k hd-256 chunk (sampled rows) passes
    the same gate; the differences between modes are logged."""
    T = 32768
    c = PrefillCase([T], [T], 8, 1, 256, seed=12)
    rows = _sample_rows(T, 32, seed=3)
    ref, slack = c.oracle(rows=rows)
    exact = c.oracle(rows=rows, exact=True)
    outs = {}
    for mode in (1, 0, 4, 32):
        log(f"prefill hd256 T={T} accum_mode={mode}")
        outs[mode] = c.run_gpu(mode)[rows]
        assert_gate(outs[mode], ref, f"accum_mode={mode}", slack=slack)
        ma, rl = metrics(outs[mode], exact)
        log(f"  vs unquantised-P reference: max_abs={ma:.3e} rel_l2={rl:.3e}")
    for mode in (0, 4, 32):
        ma, rl = metrics(outs[mode], outs[1])
        log(f"  accum_mode={mode} vs 1: max_abs={ma:.3e} rel_l2={rl:.3e}")


def test_e5m2_hd256_32k_sampled():
    # the e5m2 cache at the large-head shape and the longest single chunk
    T = 32768
    c = PrefillCase([T], [T], 8, 1, 256, seed=14, cache_dtype="e5m2")
    rows = _sample_rows(T, 48, seed=7)
    log(f"prefill e5m2 hd256 T={T} (sampled {len(rows)} rows)")
    got = c.run_gpu()
    ref, slack = c.oracle(rows=rows)
    assert_gate(got[rows], ref, f"e5m2 hd256 T={T} sampled", slack=slack)


def test_last_chunk_of_128k_fill():
    # context 131072, the last 32768 tokens are the chunk (P = 98304):
    # contraction up to 131072 keys per row, same gate
    T, L = 32768, 131072
    c = PrefillCase([T], [L], 8, 1, 256, seed=13)
    rows = _sample_rows(T, 32, seed=99)
    log(f"prefill last chunk of 128k (sampled {len(rows)} rows)")
    got = c.run_gpu()
    ref, slack = c.oracle(rows=rows)
    assert_gate(got[rows], ref, "128k fill, last 32k chunk", slack=slack)
    got0 = c.run_gpu(accum_mode=0)
    ma, rl = metrics(got0[rows], got[rows])
    log(f"  one-level vs two-level accumulation: max_abs={ma:.3e} rel_l2={rl:.3e}")


def test_empty_and_bad_arguments():
    import torch
    import attention_fp8_quantized_amd as fa
    c = PrefillCase([16], [16], 2, 1, 64, seed=1)
    d = c.dev
    with pytest.raises(fa.Fa8Error):
        fa.prefill_attention(c.q_dev, d["cu"], c.cache, d["bt"], d["lens"], d["qs"], d["ks"],
                             d["vs"], 0.125, 16, accum_mode=-1)
    # max_q_len = 0: nothing to do, nothing written
    out = torch.full((16, 2, 64), 7.0, device="cuda")
    fa.prefill_attention(c.q_dev, d["cu"], c.cache, d["bt"], d["lens"], d["qs"], d["ks"],
                         d["vs"], 0.125, 0, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
