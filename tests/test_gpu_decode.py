"""GPU split-KV decode vs the fp64 oracle.

Gate (every call): max |gpu - oracle| <= 2e-3 and relative L2 <= 1e-3 over
the compared outputs.  The same bound is used at every context length from
512 to 128k.  Large cases compare the query heads of a few KV heads (the
oracle computes those heads exactly over the whole context); the GPU runs the
full layer in the launch configuration the benchmark times (automatic split
count).
"""

import numpy as np
import pytest

from _gpu_common import DecodeCase, assert_gate, dev, log, metrics

pytestmark = pytest.mark.gpu


def _check(case, what, meta=None, **kw):
    log(f"decode {what}")
    got = case.run_gpu(**kw)
    ref, qheads = case.oracle()
    assert_gate(got[:, qheads], ref, what, meta=meta)
    return got


def test_single_layer_hd64_ctx512_unit_scales():
    # 8 q / 2 KV heads, head_dim 64, 512 tokens in 32 pages, scales 1.0
    c = DecodeCase(1, 8, 2, 64, [512], "e4m3", seed=1, scales="one")
    _check(c, "hd64 ctx512 unit scales")


@pytest.mark.parametrize("cd", ["e4m3", "e5m2", "bf16"])
@pytest.mark.parametrize("ctx", [1024, 8192, 32768, 131072])
def test_llama_shaped_layer(ctx, cd):
    # 32 q / 8 KV heads, head_dim 128, outlier channels x20, per-head absmax
    # scales (absmax/448 for e4m3, absmax/57344 for e5m2)
    heads = None if ctx <= 32768 else [0, 5]
    c = DecodeCase(1, 32, 8, 128, [ctx], cd, seed=2, outliers=True, oracle_heads=heads)
    _check(c, f"llama-shaped ctx={ctx} {cd}",
           meta=dict(kernel="decode", shape="32/8 hd128 batch 1", context=ctx, cache=cd,
                     compared=f"KV heads {heads or 'all'}"))


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("cd", ["e4m3", "e5m2", "bf16"])
def test_gqa_head_dims_ragged_batch(D, G, cd):
    Hkv = 2
    lens = [300, 0, 1, 17, 1000]
    c = DecodeCase(len(lens), G * Hkv, Hkv, D, lens, cd, seed=10 + D + G)
    got = _check(c, f"D={D} G={G} {cd} ragged")
    assert np.all(got[1] == 0), "empty sequence must give zeros"


@pytest.mark.parametrize("window", [1, 16, 100, 128, 513])
@pytest.mark.parametrize("cd", ["e4m3", "e5m2", "bf16"])
def test_sliding_window(window, cd):
    lens = [1000, 37, 128, 129]
    c = DecodeCase(len(lens), 16, 2, 64, lens, cd, seed=20 + window, window=window)
    _check(c, f"window={window} {cd}")


@pytest.mark.parametrize("cd", ["e4m3", "e5m2", "bf16"])
def test_split_count_invariance(cd):
    # Splits only regroup the same sums, but each probability is formed
    # relative to its split's running maximum, so the rounding pattern depends
    # on how tokens are grouped: the FP8 paths carry p as an f16 high + low
    # pair (about 2^-22 relative per p), the bf16 path as a bf16 high + low
    # pair (2^-18 per p, so two layouts differ by at most ~2^-17).
    c = DecodeCase(2, 32, 8, 128, [5000, 3333], cd, seed=30)
    ref, qheads = c.oracle()
    outs = {}
    for s in [1, 2, 3, 7, 0, 64, 250]:
        log(f"decode splits={s}")
        outs[s] = c.run_gpu(num_splits=s)
        assert_gate(outs[s][:, qheads], ref, f"splits={s}")
    tol = 2.0 ** -17 if cd == "bf16" else 1e-5
    for s, o in outs.items():
        ma, rl = metrics(o, outs[1])
        assert rl < tol, (s, rl)


@pytest.mark.parametrize("D,G", [(256, 4), (128, 8), (64, 16), (256, 16), (128, 16)])
def test_many_split_merge_widths(D, G):
    # Beyond 64 splits the last arrivals of every group of 16 splits each
    # merge a slice of min(128, D) columns of one query head over all the
    # set's partials (16 B per lane, 16 or 32 lanes per row slice); the sets
    # here have G*D = 1024, 2048 or 4096 outputs, so 8 to 32 slices for 7
    # or 16 groups.  With 250 splits the shorter sequence leaves most splits
    # empty; the single-split output is the reference.
    c = DecodeCase(2, 2 * G, 2, D, [3000, 1777], "e4m3", seed=40 + D + G)
    ref, qheads = c.oracle()
    one = c.run_gpu(num_splits=1)
    assert_gate(one[:, qheads], ref, f"D={D} G={G} splits=1")
    for s in [100, 250]:
        log(f"decode D={D} G={G} splits={s}")
        got = c.run_gpu(num_splits=s)
        assert_gate(got[:, qheads], ref, f"D={D} G={G} splits={s}")
        ma, rl = metrics(got, one)
        assert rl < 1e-5, (s, rl)


@pytest.mark.parametrize("cd", ["e4m3", "e5m2", "bf16"])
@pytest.mark.parametrize("window", [0, 100])
def test_stale_nan_rows_past_sequence_end(cd, window):
    # pages are pre-filled with NaN codes; the rows past each sequence end
    # keep them and must not reach the output (rows before a window start:
    # test_out_of_window_pages_never_used)
    lens = [1000, 37, 5, 129]
    c = DecodeCase(len(lens), 16, 2, 128, lens, cd, seed=33, window=window, fill=0xFF)
    got = _check(c, f"stale NaN rows {cd} window={window}")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("cd", ["e4m3", "e5m2", "bf16"])
@pytest.mark.parametrize("window", [100, 128, 513])
def test_out_of_window_pages_never_used(window, cd):
    # the cache starts as NaN codes and only the keys inside each window are
    # written: the rows before the window start in its first page keep NaN,
    # and the table entries of pages wholly before the window name a block
    # that is never written (valid memory full of NaN codes)
    lens = [1000, 37, 5, 129, 2000]
    c = DecodeCase(len(lens), 16, 2, 128, lens, cd, seed=50 + window, window=window,
                   fill=0xFF, window_only=True)
    got = _check(c, f"out-of-window NaN pages {cd} window={window}")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("cd", ["e4m3", "e5m2", "bf16"])
@pytest.mark.parametrize("in_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("window", [0, 100])
def test_fused_append_equals_write_then_decode(cd, in_dtype, window):
    # the current token's K/V is written by the decode launch itself: the cache
    # bytes and the output must equal cache_write followed by decode
    import torch
    import attention_fp8_quantized_amd as fa
    lens = [300, 1, 17, 1000, 16, 0]
    c = DecodeCase(len(lens), 16, 2, 128, lens, cd, seed=34, window=window, skip_last=True,
                   fill=0xFF)
    tdt = torch.bfloat16 if in_dtype == "bf16" else torch.float32
    B, Hkv, D = c.B, c.Hkv, c.D
    k_new = np.zeros((B, Hkv, D), np.float32)
    v_new = np.zeros((B, Hkv, D), np.float32)
    has = c.lens > 0
    k_new[has] = c.k[c.last_idx]
    v_new[has] = c.v[c.last_idx]
    kd, vd = dev(k_new).to(tdt), dev(v_new).to(tdt)
    start = c.cache.clone()
    # write, then decode
    sl = np.where(has, c.bt[np.arange(B), np.maximum(c.lens - 1, 0) // 16] * 16 +
                  np.maximum(c.lens - 1, 0) % 16, -1).astype(np.int64)
    fa.cache_write(kd, vd, dev(sl), c.ks_dev, c.vs_dev, c.cache)
    ref_out = c.run_gpu()
    ref_cache = c.cache.clone()
    # fused
    c.cache.copy_(start)
    log(f"decode fused append {cd} in={in_dtype} window={window}")
    out = fa.decode_attention_append(c.q_dev, kd, vd, c.cache, c.bt_dev, c.lens_dev, c.ks_dev,
                                     c.vs_dev, float(c.sm), int(c.lens.max()), window=window)
    torch.cuda.synchronize()
    assert torch.equal(c.cache.view(torch.uint8), ref_cache.view(torch.uint8)), "cache bytes"
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got, ref_out)
    if in_dtype == "fp32":
        ref, qheads = c.oracle()
        assert_gate(got[:, qheads], ref, f"fused append {cd} window={window}")


def test_page_permutation_invariance():
    import torch
    c = DecodeCase(1, 32, 8, 128, [4000], "e4m3", seed=31)
    base = c.run_gpu()
    # move every physical block to a new id and rewrite the table
    nb = c.cache.shape[0]
    perm = torch.from_numpy(np.random.default_rng(0).permutation(nb)).cuda()
    moved = torch.empty_like(c.cache)
    moved[perm] = c.cache
    c.cache = moved
    bt = c.bt.copy()
    bt[bt >= 0] = perm.cpu().numpy()[bt[bt >= 0]]
    c.bt_dev = torch.from_numpy(bt).cuda()
    log("decode page permutation")
    got = c.run_gpu()
    np.testing.assert_array_equal(got, base)


def test_uniform_scores_give_mean_of_v():
    # q = 0: every visible token has weight 1/n, so out = mean of V-hat
    from oracle import e4m3
    c = DecodeCase(2, 8, 2, 128, [777, 64], "e4m3", seed=32, q_zero=True)
    got = c.run_gpu()
    at = 0
    for b, L in enumerate(c.lens):
        for hq in range(8):
            h = hq // 4
            codes = np.array([np.frombuffer(e4m3.encode(c.v[at + t, h] / c.vs[h]).tobytes(), np.uint8)
                              for t in range(L)])
            mean = e4m3.decode(codes).mean(axis=0) * np.float64(c.vs[h])
            ma, rl = metrics(got[b, hq], mean)
            assert ma < 1e-5 and rl < 1e-5, (b, hq, ma, rl)
        at += L


def test_more_sets_than_compute_units():
    # 40 sequences x 8 KV heads = 320 (sequence, KV head) sets: one split
    # each, so the workgroups run in more than one round and write their rows
    # straight from the wave merge; ragged lengths, one empty sequence
    import attention_fp8_quantized_amd as fa
    rng = np.random.default_rng(60)
    lens = [int(x) for x in rng.integers(1, 600, size=40)]
    lens[3] = 0
    assert fa.decode_num_splits(40, 8, max(lens)) == 1
    c = DecodeCase(40, 32, 8, 128, lens, "e4m3", seed=60)
    got = _check(c, "40 sequences x 8 KV heads, one split")
    assert np.all(got[3] == 0), "empty sequence must give zeros"
    # and with explicit splits: 320 sets x 4 splits, four rounds of workgroups
    got4 = c.run_gpu(num_splits=4)
    ref, qheads = c.oracle()
    assert_gate(got4[:, qheads], ref, "40 sequences x 8 KV heads, 4 splits")


def test_loaded_decode_shape():
    # 8 sequences of U{18000..22000} tokens, 32 q / 8 KV heads, head_dim 128
    import workloads as W
    lens = W.uniform_lengths(W.rng(3, 0, W.LENGTHS), 8, 18000, 22000)
    c = DecodeCase(8, 32, 8, 128, lens, "e4m3", seed=3, oracle_heads=[3])
    _check(c, "8 x ~20k loaded decode")


@pytest.mark.parametrize("variant", ["full-fp8", "sw128-bf16", "sw128-fp8"])
def test_hybrid_layers(variant):
    # gpt-oss-20b-shaped: 64 q / 8 KV heads, head_dim 64, 8 x 20000 tokens
    cd = "bf16" if "bf16" in variant else "e4m3"
    window = 128 if variant.startswith("sw") else 0
    heads = [1] if window == 0 else None
    c = DecodeCase(8, 64, 8, 64, [20000] * 8, cd, seed=4, window=window, oracle_heads=heads)
    _check(c, f"hybrid {variant}")


@pytest.mark.parametrize("ctx", [1024, 8192, 32768, 131072])
def test_hd256_long_decode(ctx):
    # 8 q / 1 KV head, head_dim 256, per-head absmax scales, contexts to 128k
    c = DecodeCase(1, 8, 1, 256, [ctx], "e4m3", seed=5)
    _check(c, f"hd256 ctx={ctx}",
           meta=dict(kernel="decode", shape="8/1 hd256 batch 1", context=ctx, cache="e4m3",
                     compared="all heads"))


def test_argument_errors_raise():
    import torch
    import attention_fp8_quantized_amd as fa
    c = DecodeCase(1, 8, 2, 64, [64], "e4m3", seed=6)
    with pytest.raises(fa.Fa8Error):
        # workspace far too small
        fa.decode_attention(c.q_dev, c.cache, c.bt_dev, c.lens_dev, c.ks_dev, c.vs_dev,
                            0.125, 64, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(fa.Fa8Error):
        # max_seq_len beyond what the block table can address
        fa.decode_attention(c.q_dev, c.cache, c.bt_dev, c.lens_dev, c.ks_dev, c.vs_dev,
                            0.125, 10 ** 6)


def test_fused_append_full_size_llama_32k():
    """The benchmark's step configuration: one 32k-token Llama-shaped layer
    (32 q / 8 KV heads, head_dim 128, outlier channels), the library's split
    count.  The fused launch must leave the same cache bytes and the same
    output as cache_write followed by decode, and match the oracle on two
    KV heads."""
    import torch
    import attention_fp8_quantized_amd as fa
    L = 32768
    c = DecodeCase(1, 32, 8, 128, [L], "e4m3", seed=35, outliers=True, skip_last=True,
                   oracle_heads=[2, 7])
    k_new = dev(c.k[c.last_idx])
    v_new = dev(c.v[c.last_idx])
    slot = int(c.bt[0, (L - 1) // 16]) * 16 + (L - 1) % 16
    start = c.cache.clone()
    fa.cache_write(k_new, v_new, dev(np.array([slot], np.int64)), c.ks_dev, c.vs_dev, c.cache)
    ref_out = c.run_gpu()
    ref_cache = c.cache.clone()
    c.cache.copy_(start)
    log("decode fused append, 32k Llama-shaped layer")
    out = fa.decode_attention_append(c.q_dev, k_new, v_new, c.cache, c.bt_dev, c.lens_dev,
                                     c.ks_dev, c.vs_dev, float(c.sm), L)
    torch.cuda.synchronize()
    assert torch.equal(c.cache.view(torch.uint8), ref_cache.view(torch.uint8)), "cache bytes"
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got, ref_out)
    ref, qheads = c.oracle()
    assert_gate(got[:, qheads], ref, "fused append 32k")
