"""GPU FP8 prefill vs the tile-mirrored fp64 oracle.

The oracle quantises P exactly where the method does (per 128-key tile at
absolute aligned positions, against the running row maximum after that tile)
and keeps the softmax denominator unquantised.  Gate: max |gpu - oracle| <=
2e-3 and relative L2 <= 1e-3 over the compared rows, the same bound from 200
to 131072 keys.  The unquantised-P reference (prefill_exact) is reported.
Large cases compare 64 sampled rows per chunk: the last 16 and 48 seeded
random rows.  Every gated comparison is recorded (FA8_PARITY_LOG) with its
shape, context and accumulation mode.
"""

import numpy as np
import pytest

from _gpu_common import PrefillCase, assert_gate, log, metrics

pytestmark = pytest.mark.gpu


def _sample_rows(T, seed, n=64):
    """The last 16 rows of a chunk plus n - 16 seeded random rows before them."""
    g = np.random.default_rng(seed)
    tail = np.arange(max(0, T - 16), T)
    rest = g.choice(max(T - 16, 1), size=min(n - len(tail), max(T - 16, 0)), replace=False)
    return np.unique(np.concatenate([rest, tail])).astype(np.int64)


def _meta(D, heads, T, L, mode, cd="e4m3", rows="all"):
    return dict(kernel="prefill", shape=f"{heads} hd{D}", chunk=T, context=L, accum_mode=mode,
                cache=cd, compared=rows)


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


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("cd", ["e4m3", "e5m2"])
@pytest.mark.parametrize("window", [0, 100])
def test_chunked_ragged_batch_gqa(window, cd, D):
    # three sequences: fresh (P=0), continued (P=300), short tail chunk; at
    # head_dim 64 and 256 the workgroups hold 64 rows and one tile buffer
    c = PrefillCase([130, 100, 17], [130, 400, 260], 8, 2, D, seed=7, window=window,
                    cache_dtype=cd)
    log(f"prefill ragged window={window} cache={cd} D={D}")
    ref, slack = c.oracle()
    assert_gate(c.run_gpu(), ref, f"ragged batch window={window} {cd} D={D}", slack=slack)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_chunk_lengths_around_workgroup_rows(D):
    # chunk lengths one below, at and one above the 64- and 128-row query
    # blocks, fresh and continued sequences
    c = PrefillCase([63, 64, 65, 127, 128, 129], [63, 200, 65, 300, 128, 700], 4, 2, D,
                    seed=80 + D)
    log(f"prefill chunk lengths around the query blocks D={D}")
    ref, slack = c.oracle()
    assert_gate(c.run_gpu(), ref, f"chunk lengths around the query blocks D={D}", slack=slack)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("window", [0, 100])
def test_one_and_two_query_chunks(D, window):
    # a chunk of one or two queries deep in its sequence: one query block,
    # nearly all of its rows past the chunk end
    c = PrefillCase([1, 1, 2], [1, 517, 260], 4, 2, D, seed=90 + D + window, window=window)
    log(f"prefill one- and two-query chunks D={D} window={window}")
    ref, slack = c.oracle()
    assert_gate(c.run_gpu(), ref, f"one- and two-query chunks D={D} window={window}", slack=slack)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("cd", ["e4m3", "e5m2"])
def test_stale_nan_rows_past_sequence_end(cd, D):
    # pages are pre-filled with NaN codes (0xFF in both FP8 formats); the rows
    # past each sequence end keep them and must not reach the output
    c = PrefillCase([130, 75], [130, 333], 4, 2, D, seed=8, fill=0xFF, cache_dtype=cd)
    log(f"prefill stale NaN rows cache={cd} D={D}")
    got = c.run_gpu()
    assert np.all(np.isfinite(got))
    ref, slack = c.oracle()
    assert_gate(got, ref, "stale NaN rows", slack=slack)


@pytest.mark.parametrize("cd", ["e4m3", "e5m2"])
@pytest.mark.parametrize("window", [100, 128, 513])
def test_out_of_window_pages_never_used(window, cd):
    # the cache starts as NaN codes and only keys some query can see are
    # written (from the first query's window start on); the table entries of
    # pages wholly before that name a block that is never written.  Chunks
    # sit deep in their sequences, so a workgroup's first staged tile starts
    # before its window
    c = PrefillCase([200, 130, 17], [1000, 700, 260], 8, 2, 128, seed=60 + window,
                    window=window, fill=0xFF, cache_dtype=cd, window_only=True)
    log(f"prefill out-of-window NaN pages window={window} cache={cd}")
    got = c.run_gpu()
    assert np.all(np.isfinite(got))
    ref, slack = c.oracle()
    assert_gate(got, ref, f"out-of-window NaN pages window={window} {cd}", slack=slack)


@pytest.mark.parametrize("D", [64, 256])
def test_out_of_window_pages_never_used_head_dims(D):
    c = PrefillCase([300, 129], [2000, 4096], 8, 1, D, seed=70 + D, window=513, fill=0xFF,
                    window_only=True)
    log(f"prefill out-of-window NaN pages D={D} window=513")
    got = c.run_gpu()
    assert np.all(np.isfinite(got))
    ref, slack = c.oracle()
    assert_gate(got, ref, f"out-of-window NaN pages D={D}", slack=slack)


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
    assert_gate(c.run_gpu(accum_mode), ref, f"hd256 T=1024 accum={accum_mode}", slack=slack,
                meta=_meta(256, "8/1", 1024, 1024, accum_mode))


@pytest.mark.parametrize("T", [8192, 32768])
def test_hd256_long_chunk_sampled(T):
    # two-level and one-level accumulation against the same mirror
    c = PrefillCase([T], [T], 8, 1, 256, seed=12)
    rows = _sample_rows(T, seed=T)
    ref, slack = c.oracle(rows=rows)
    for mode in (1, 0):
        log(f"prefill hd256 T={T} accum_mode={mode} (sampled {len(rows)} rows)")
        got = c.run_gpu(mode)
        assert_gate(got[rows], ref, f"hd256 T={T} accum={mode} sampled", slack=slack,
                    meta=_meta(256, "8/1", T, T, mode, rows=f"{len(rows)} sampled rows"))


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (32, 8)])
def test_hd128_32k_chunk_sampled(Hq, Hkv):
    # head_dim 128 over a 32k contraction (Llama-shaped 32/8 and 8/1 heads)
    T = 32768
    c = PrefillCase([T], [T], Hq, Hkv, 128, seed=16 + Hkv)
    rows = _sample_rows(T, seed=17)
    ref, slack = c.oracle(rows=rows)
    for mode in (1, 0):
        log(f"prefill hd128 {Hq}/{Hkv} T={T} accum_mode={mode} (sampled {len(rows)} rows)")
        got = c.run_gpu(mode)
        assert_gate(got[rows], ref, f"hd128 {Hq}/{Hkv} T={T} accum={mode} sampled", slack=slack,
                    meta=_meta(128, f"{Hq}/{Hkv}", T, T, mode, rows=f"{len(rows)} sampled rows"))


@pytest.mark.parametrize("T", [1024, 8192, 32768])
def test_hd64_long_chunk_sampled(T):
    c = PrefillCase([T], [T], 8, 1, 64, seed=18)
    rows = _sample_rows(T, seed=19) if T > 1024 else None
    ref, slack = c.oracle(rows=rows)
    log(f"prefill hd64 T={T}")
    got = c.run_gpu()
    sel = got if rows is None else got[rows]
    assert_gate(sel, ref, f"hd64 8/1 T={T}", slack=slack,
                meta=_meta(64, "8/1", T, T, 1,
                           rows="all" if rows is None else f"{len(rows)} sampled rows"))


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
    rows = _sample_rows(T, seed=3)
    ref, slack = c.oracle(rows=rows)
    exact = c.oracle(rows=rows, exact=True)
    outs = {}
    for mode in (1, 0, 4, 32):
        log(f"prefill hd256 T={T} accum_mode={mode}")
        outs[mode] = c.run_gpu(mode)[rows]
        assert_gate(outs[mode], ref, f"accum_mode={mode}", slack=slack,
                    meta=_meta(256, "8/1", T, T, mode, rows=f"{len(rows)} sampled rows"))
        ma, rl = metrics(outs[mode], exact)
        log(f"  vs unquantised-P reference: max_abs={ma:.3e} rel_l2={rl:.3e}")
    for mode in (0, 4, 32):
        ma, rl = metrics(outs[mode], outs[1])
        log(f"  accum_mode={mode} vs 1: max_abs={ma:.3e} rel_l2={rl:.3e}")


def test_e5m2_hd256_32k_sampled():
    # the e5m2 cache at the large-head shape and the longest single chunk
    T = 32768
    c = PrefillCase([T], [T], 8, 1, 256, seed=14, cache_dtype="e5m2")
    rows = _sample_rows(T, seed=7)
    log(f"prefill e5m2 hd256 T={T} (sampled {len(rows)} rows)")
    got = c.run_gpu()
    ref, slack = c.oracle(rows=rows)
    assert_gate(got[rows], ref, f"e5m2 hd256 T={T} sampled", slack=slack,
                meta=_meta(256, "8/1", T, T, 1, cd="e5m2", rows=f"{len(rows)} sampled rows"))


def test_last_chunk_of_128k_fill():
    # context 131072, the last 32768 tokens are the chunk (P = 98304):
    # contraction up to 131072 keys per row, same gate
    T, L = 32768, 131072
    c = PrefillCase([T], [L], 8, 1, 256, seed=13)
    rows = _sample_rows(T, seed=99)
    ref, slack = c.oracle(rows=rows)
    outs = {}
    for mode in (1, 0):
        log(f"prefill last chunk of 128k accum_mode={mode} (sampled {len(rows)} rows)")
        outs[mode] = c.run_gpu(accum_mode=mode)[rows]
        assert_gate(outs[mode], ref, f"128k fill, last 32k chunk, accum={mode}", slack=slack,
                    meta=_meta(256, "8/1", T, L, mode, rows=f"{len(rows)} sampled rows"))
    ma, rl = metrics(outs[0], outs[1])
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
