"""Pins of the oracle's cache write, decode and prefill references (CPU only).

Pins used (none re-types the oracle's own formula):
* literal Python triple loops over tiny inputs (math.exp, explicit indexing);
* closed forms: uniform scores give the mean of V; one key gives V itself;
  a dominant "needle" key gives its own V;
* a second formulation (random splits + log-sum-exp merge);
* structural invariances: page permutation, windowing == truncation;
* a hand-worked tile example (tests/golden/prefill_mirror_tiny.json).
"""

import json
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import quant as Qn
from oracle import e4m3, e5m2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(B=2, Hq=8, Hkv=2, D=64, lens=(37, 20), cache_dtype="e4m3", seed=0,
          scale_kind="absmax"):
    g = np.random.default_rng(seed)
    lens = np.array(lens, dtype=np.int32)
    bt, nblocks = W.block_table(g, lens)
    N = int(lens.sum())
    k = W.normal(g, (N, Hkv, D))
    v = W.normal(g, (N, Hkv, D))
    if scale_kind == "absmax":
        ks, vs = W.absmax_scales(k), W.absmax_scales(v)
    else:
        ks = vs = np.ones(Hkv, dtype=np.float32)
    slots = W.all_slots(bt, lens)
    cache = Qn.new_cache(nblocks, Hkv, D, cache_dtype)
    Qn.cache_write(cache, k, v, slots, ks, vs, cache_dtype)
    _, q = W.bf16_values(W.normal(g, (B, Hq, D)))
    return dict(q=q, cache=cache, bt=bt, lens=lens, ks=ks, vs=vs, k=k, v=v,
                Hkv=Hkv, D=D, cd=cache_dtype)


# ----------------------------------------------------------------------------
# cache write
# ----------------------------------------------------------------------------

def test_cache_write_layout_by_hand():
    Hkv, D = 2, 4
    cache = Qn.new_cache(3, Hkv, D, "e4m3", fill=0xA5)
    k = np.arange(2 * Hkv * D, dtype=np.float32).reshape(2, Hkv, D)   # exact codes
    v = -k
    one = np.ones(Hkv, dtype=np.float32)
    Qn.cache_write(cache, k, v, np.array([17, -1]), one, one, "e4m3")
    # slot 17 -> block 1, row 1;  the second row is padding (slot -1)
    for h in range(Hkv):
        for d in range(D):
            assert cache[1, h, 0, 1, d] == e4m3.encode(np.float32(k[0, h, d]))
            assert cache[1, h, 1, 1, d] == e4m3.encode(np.float32(-k[0, h, d]))
    touched = np.zeros(cache.shape, dtype=bool)
    touched[1, :, :, 1, :] = True
    assert np.all(cache[~touched] == 0xA5)


def test_cache_write_scale_divides():
    # x / s with s a power of two moves codes by whole binades
    k = np.full((1, 1, 8), 3.0, dtype=np.float32)
    c1 = Qn.new_cache(1, 1, 8, "e4m3")
    c2 = Qn.new_cache(1, 1, 8, "e4m3")
    Qn.cache_write(c1, k, k, np.array([0]), np.array([1.0], np.float32),
                   np.array([1.0], np.float32), "e4m3")
    Qn.cache_write(c2, k, k, np.array([0]), np.array([0.5], np.float32),
                   np.array([4.0], np.float32), "e4m3")
    assert e4m3.decode(c1[0, 0, 0, 0, 0]) == 3.0
    assert e4m3.decode(c2[0, 0, 0, 0, 0]) == 6.0      # 3 / 0.5
    assert e4m3.decode(c2[0, 0, 1, 0, 0]) == 0.75     # 3 / 4


def _division_golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "quantize_division.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        fmt, rest = line.split(None, 1)
        *xe, se, code = rest.split()
        rows.append((fmt, np.float32(eval(" ".join(xe))), np.float32(float(se)), int(code, 16)))
    return rows


def _quantize_by_reciprocal(x, s, fmt):
    """A plausible wrong reading: multiply by the fp32 reciprocal of the
    scale instead of dividing by it."""
    r = np.float32(np.float32(1.0) / np.float32(s))
    y = np.multiply(np.float32(x), r, dtype=np.float32)
    return (e4m3.encode(y) if fmt == "e4m3" else e5m2.encode(y))


def test_quantize_rows_divides_correctly_rounded():
    # hand-worked rows on FP8 rounding midpoints (tests/golden/quantize_division.txt)
    rows = _division_golden()
    assert len(rows) >= 3
    separating = 0
    for fmt, x, s, code in rows:
        got = int(Qn.quantize_rows(np.array([x]), s, fmt)[0])
        assert got == code, (fmt, float(x), float(s), hex(got), hex(code))
        # the same value through the cache write, as a K row of head 0
        c = Qn.new_cache(1, 1, 1, fmt)
        Qn.cache_write(c, np.array([[[x]]]), np.array([[[x]]]), np.array([3]),
                       np.array([s]), np.array([s]), fmt)
        assert c[0, 0, 0, 3, 0] == code and c[0, 0, 1, 3, 0] == code
        if int(_quantize_by_reciprocal(x, s, fmt)) != code:
            separating += 1
    # the reciprocal-multiply reading fails every midpoint row at s = 7
    assert separating == sum(1 for r in rows if r[2] == np.float32(7.0)) >= 3


def test_e5m2_cache_write_layout_and_scale():
    Hkv, D = 2, 4
    cache = Qn.new_cache(3, Hkv, D, "e5m2", fill=0xA5)
    k = np.arange(2 * Hkv * D, dtype=np.float32).reshape(2, Hkv, D) * np.float32(1000.0)
    v = -k
    ks = np.array([0.5, 1.0], np.float32)
    vs = np.array([4.0, 2.0], np.float32)
    Qn.cache_write(cache, k, v, np.array([-1, 33]), ks, vs, "e5m2")
    # slot 33 -> block 2, row 1;  the first row is padding (slot -1)
    for h in range(Hkv):
        for d in range(D):
            assert cache[2, h, 0, 1, d] == e5m2.encode(np.float32(k[1, h, d] / ks[h]))
            assert cache[2, h, 1, 1, d] == e5m2.encode(np.float32(-k[1, h, d] / vs[h]))
    touched = np.zeros(cache.shape, dtype=bool)
    touched[2, :, :, 1, :] = True
    assert np.all(cache[~touched] == 0xA5)
    # by hand: head 1, channel 3 holds 15000 / 1.0; the e5m2 grid in
    # [8192, 16384) has step 2048, so the nearest value is 14336.  Head 0,
    # channel 3 holds 11000 / 0.5 = 22000; step 4096 in [16384, 32768): 20480
    assert e5m2.decode(cache[2, 1, 0, 1, 3]) == 14336.0
    assert e5m2.decode(cache[2, 0, 0, 1, 3]) == 20480.0
    # dequantisation multiplies back by the scale
    assert Qn.dequantize(cache[2, 0, 0, 1, 3], ks[0], "e5m2") == 10240.0


def test_bf16_cache_ignores_scales():
    g = np.random.default_rng(1)
    k = g.standard_normal((3, 2, 8)).astype(np.float32)
    c = Qn.new_cache(1, 2, 8, "bf16")
    Qn.cache_write(c, k, k, np.array([0, 5, 9]), np.array([7.0, 7.0], np.float32),
                   np.array([7.0, 7.0], np.float32), "bf16")
    import torch
    ref = torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(c[0, :, 0, [0, 5, 9], :], ref)


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

def _literal_decode(q, cache, bt, lens, ks, vs, sm, window, Hkv, cd):
    """Triple loop, math.exp, explicit page indexing."""
    B, Hq, D = q.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lens[b])
        lo = max(0, L - window) if window > 0 else 0
        for hq in range(Hq):
            h = hq // G
            scores = []
            vals = []
            for t in range(lo, L):
                blk = int(bt[b][t // 16])
                row = t % 16
                if cd in ("e4m3", "e5m2"):
                    dc = e4m3.decode_code if cd == "e4m3" else e5m2.decode_code
                    kv = [float(ks[h]) * dc(int(cache[blk, h, 0, row, d])) for d in range(D)]
                    vv = [float(vs[h]) * dc(int(cache[blk, h, 1, row, d])) for d in range(D)]
                else:
                    kv = [float(np.uint32(int(cache[blk, h, 0, row, d]) << 16).view(np.float32)) for d in range(D)]
                    vv = [float(np.uint32(int(cache[blk, h, 1, row, d]) << 16).view(np.float32)) for d in range(D)]
                s = 0.0
                for d in range(D):
                    s += float(q[b, hq, d]) * kv[d]
                scores.append(float(np.float32(sm)) * s)
                vals.append(vv)
            if not scores:
                continue
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for d in range(D):
                out[b, hq, d] = sum(w[j] * vals[j][d] for j in range(len(w))) / tot
    return out


@pytest.mark.parametrize("cd", ["e4m3", "e5m2", "bf16"])
@pytest.mark.parametrize("window", [0, 7])
def test_decode_vs_literal_loop(cd, window):
    c = _case(B=2, Hq=4, Hkv=2, D=8, lens=(37, 5), cache_dtype=cd, seed=3)
    sm = np.float32(1 / math.sqrt(8))
    got = A.decode_attention(c["q"], c["cache"], c["bt"], c["lens"], c["ks"], c["vs"],
                             sm, window, cd, c["Hkv"])
    ref = _literal_decode(c["q"], c["cache"], c["bt"], c["lens"], c["ks"], c["vs"],
                          sm, window, c["Hkv"], cd)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_decode_uniform_scores_is_mean_of_v():
    c = _case(lens=(45, 16), seed=4)
    q0 = np.zeros_like(c["q"])
    for window in (0, 10):
        got = A.decode_attention(q0, c["cache"], c["bt"], c["lens"], c["ks"], c["vs"],
                                 0.125, window, "e4m3", c["Hkv"])
        G = q0.shape[1] // c["Hkv"]
        for b, L in enumerate(c["lens"]):
            lo = max(0, L - window) if window else 0
            for hq in range(q0.shape[1]):
                h = hq // G
                # V-hat of every visible token, straight from the fp32 inputs'
                # codes: decode(code) * scale; mean over tokens
                toks = [int(c["bt"][b][t // 16]) for t in range(lo, L)]
                rows = [t % 16 for t in range(lo, L)]
                vhat = np.array([e4m3.decode(c["cache"][blk, h, 1, r, :]) for blk, r in zip(toks, rows)])
                np.testing.assert_allclose(got[b, hq], vhat.mean(axis=0) * c["vs"][h], rtol=1e-13)


def test_decode_single_token_returns_v0():
    c = _case(B=1, lens=(1,), seed=5)
    got = A.decode_attention(c["q"], c["cache"], c["bt"], c["lens"], c["ks"], c["vs"],
                             0.125, 0, "e4m3", c["Hkv"])
    blk = c["bt"][0][0]
    for hq in range(c["q"].shape[1]):
        h = hq // 4
        np.testing.assert_array_equal(got[0, hq], e4m3.decode(c["cache"][blk, h, 1, 0]) * np.float64(c["vs"][h]))


def test_decode_empty_sequence_is_zero():
    c = _case(B=2, lens=(0, 9), seed=6)
    got = A.decode_attention(c["q"], c["cache"], c["bt"], c["lens"], c["ks"], c["vs"],
                             0.125, 0, "e4m3", c["Hkv"])
    assert np.all(got[0] == 0)
    assert np.all(np.isfinite(got[1]))


def test_decode_needle():
    # q parallel to the needle key and scaled up: all weight on that token
    c = _case(B=1, Hq=2, Hkv=1, D=64, lens=(300,), seed=8)
    n = 123
    blk, row = c["bt"][0][n // 16], n % 16
    kn = e4m3.decode(c["cache"][blk, 0, 0, row]) * c["ks"][0]
    q = (kn / np.linalg.norm(kn) * 400.0)[None, None, :].repeat(2, axis=1)
    got = A.decode_attention(q, c["cache"], c["bt"], c["lens"], c["ks"], c["vs"],
                             1.0, 0, "e4m3", 1)
    want = e4m3.decode(c["cache"][blk, 0, 1, row]) * c["vs"][0]
    np.testing.assert_allclose(got[0, 0], want, atol=1e-6)


@pytest.mark.parametrize("window", [0, 33])
def test_decode_split_lse_formulation_agrees(window):
    c = _case(B=2, Hq=8, Hkv=2, D=32, lens=(300, 97), seed=9)
    args = (c["q"], c["cache"], c["bt"], c["lens"], c["ks"], c["vs"], 0.2, window, "e4m3", 2)
    direct = A.decode_attention(*args)
    for s in range(3):
        split = A.decode_attention_split(*args, rng=np.random.default_rng(s))
        np.testing.assert_allclose(split, direct, rtol=1e-12, atol=1e-14)


def test_decode_page_permutation_invariance():
    c = _case(B=1, lens=(200,), seed=10)
    base = A.decode_attention(c["q"], c["cache"], c["bt"], c["lens"], c["ks"], c["vs"],
                              0.125, 0, "e4m3", c["Hkv"])
    perm = np.random.default_rng(0).permutation(c["cache"].shape[0])
    cache2 = np.empty_like(c["cache"])
    cache2[perm] = c["cache"]                 # block i moves to perm[i]
    bt2 = c["bt"].copy()
    used = bt2 >= 0
    bt2[used] = perm[bt2[used]]
    got = A.decode_attention(c["q"], cache2, bt2, c["lens"], c["ks"], c["vs"],
                             0.125, 0, "e4m3", c["Hkv"])
    np.testing.assert_array_equal(got, base)


def test_window_equals_truncated_sequence():
    # attention over the last w tokens == full attention over a sequence
    # that holds only those w tokens
    g = np.random.default_rng(12)
    L, w, Hkv, D = 90, 25, 1, 16
    k = W.normal(g, (L, Hkv, D))
    v = W.normal(g, (L, Hkv, D))
    one = np.ones(1, np.float32)
    bt_full = np.arange(6, dtype=np.int32)[None, :]
    c_full = Qn.cache_write(Qn.new_cache(6, Hkv, D, "e4m3"), k, v, np.arange(L), one, one, "e4m3")
    bt_tail = np.arange(2, dtype=np.int32)[None, :]
    c_tail = Qn.cache_write(Qn.new_cache(2, Hkv, D, "e4m3"), k[L - w:], v[L - w:],
                            np.arange(w), one, one, "e4m3")
    _, q = W.bf16_values(W.normal(g, (1, 2, D)))
    a = A.decode_attention(q, c_full, bt_full, [L], one, one, 0.25, w, "e4m3", 1)
    b = A.decode_attention(q, c_tail, bt_tail, [w], one, one, 0.25, 0, "e4m3", 1)
    np.testing.assert_allclose(a, b, rtol=1e-13)


def test_lse_combine_edge_cases():
    o = np.array([[1.0, 2.0], [3.0, 4.0]])
    assert np.all(A.lse_combine(o, [-np.inf, -np.inf], [0, 0]) == 0)
    np.testing.assert_allclose(A.lse_combine(o, [0.0, -np.inf], [2.0, 0.0]), [0.5, 1.0])
    # equal maxima: plain sum / sum
    np.testing.assert_allclose(A.lse_combine(o, [1.0, 1.0], [1.0, 3.0]), [1.0, 1.5])


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------

def test_mirror_tiny_worked_example():
    with open(os.path.join(GOLDEN, "prefill_mirror_tiny.json")) as f:
        ex = json.load(f)
    s = np.array([eval(x, {"math": math}) for x in ex["scores"]])
    keys = np.array(ex["keys"])
    V = np.array(ex["values"])[:, None]
    got_q = A.mirror_row(s, keys, V, ex["kv_tile"], quantize_p=True)[0]
    got_x = A.mirror_row(s, keys, V, ex["kv_tile"], quantize_p=False)[0]
    assert got_q == pytest.approx(eval(ex["expected_quantized"]), rel=1e-15)
    assert got_x == pytest.approx(eval(ex["expected_exact"]), rel=1e-15)


def _window_relative_mirror(s, keys, V, kv_tile, quantize_p=True):
    """A plausible wrong reading: tiles counted from the first visible key."""
    return A.mirror_row(s, keys - keys[0], V, kv_tile, quantize_p)


def test_mirror_windowed_rows_use_absolute_tiles():
    # hand-worked rows whose first visible key is not tile-aligned
    # (tests/golden/prefill_mirror_window.json), including the kernel's
    # 128-key tile width
    with open(os.path.join(GOLDEN, "prefill_mirror_window.json")) as f:
        ex = json.load(f)
    s = np.array([eval(x, {"math": math}) for x in ex["scores"]])
    V = np.array(ex["values"])[:, None]
    want_q = eval(ex["expected_quantized"])
    want_rel = eval(ex["expected_window_relative_tiles"])
    assert abs(want_q - want_rel) > 1e-3
    for case in ex["cases"]:
        keys = np.array(case["keys"])
        bn = case["kv_tile"]
        assert keys[0] % bn != 0
        assert A.mirror_row(s, keys, V, bn)[0] == pytest.approx(want_q, rel=1e-14)
        assert A.recurrence_row(s, keys, V, bn) == pytest.approx(np.array([want_q]), rel=1e-14)
        assert A.mirror_row(s, keys, V, bn, quantize_p=False)[0] == pytest.approx(
            eval(ex["expected_exact"]), rel=1e-14)
        # the window-relative reading lands on the other value, so it fails
        rel = _window_relative_mirror(s, keys, V, bn)[0]
        assert rel == pytest.approx(want_rel, rel=1e-14)
        assert rel != pytest.approx(want_q, rel=1e-6)


def test_windowed_prefill_mirror_passes_absolute_key_positions():
    # through the whole reference (cache, block table, masks): every row of a
    # windowed chunk equals mirror_row over its visible keys at their absolute
    # positions; with the window start inside a tile, tiles counted from the
    # window start give a different result for some row
    kv_tile = 16
    c = _case(B=1, Hq=2, Hkv=1, D=64, lens=(90,), seed=21)
    q = W.bf16_values(W.normal(np.random.default_rng(5), (40, 2, 64)))[1]
    cu = np.array([0, 40], np.int32)
    qs = np.float32(np.abs(q).max() / 448.0)
    sm = np.float32(0.125)
    window = 37                                    # starts are not 16-aligned
    out = A.prefill_mirror(q, cu, c["cache"], c["bt"], c["lens"], qs, c["ks"], c["vs"],
                           sm, window, kv_tile)
    K, Vv = A.gather_kv(c["cache"], c["bt"][0], 0, 90, 0, "e4m3", c["ks"], c["vs"])
    qhat = A.quantize_query(q, qs)
    differs = 0
    for r in range(40):
        pos = 50 + r
        lo, hi = A.visible_range(pos, window)
        keys = np.arange(lo, hi)
        for hq in range(2):
            sc = np.float64(sm) * (qhat[r, hq] @ K[lo:hi].T)
            want = A.mirror_row(sc, keys, Vv[lo:hi], kv_tile)
            np.testing.assert_allclose(out[r, hq], want, rtol=0, atol=1e-13)
            wrong = _window_relative_mirror(sc, keys, Vv[lo:hi], kv_tile)
            differs += int(np.max(np.abs(wrong - want)) > 1e-9)
    assert differs > 0


@pytest.mark.parametrize("kv_tile", [2, 16, 64])
def test_mirror_closed_form_equals_literal_recurrence(kv_tile):
    g = np.random.default_rng(kv_tile)
    for lo, hi in [(0, 40), (5, 77), (31, 33)]:
        keys = np.arange(lo, hi)
        s = g.standard_normal(len(keys)) * 3
        V = g.standard_normal((len(keys), 5))
        for qp in (True, False):
            np.testing.assert_allclose(A.mirror_row(s, keys, V, kv_tile, qp),
                                       A.recurrence_row(s, keys, V, kv_tile, qp),
                                       rtol=1e-12, atol=1e-14)


def test_mirror_single_tile_quantizes_final_max():
    g = np.random.default_rng(2)
    keys = np.arange(0, 50)
    s = g.standard_normal(50) * 2
    V = g.standard_normal((50, 3))
    p = np.exp(s - s.max())
    pq = np.array([e4m3.decode_code(int(e4m3.encode(np.array([x]))[0])) for x in p])
    want = (pq @ V) / p.sum()
    np.testing.assert_allclose(A.mirror_row(s, keys, V, 64), want, rtol=1e-13)


def _prefill_case(T=40, P=0, Hq=4, Hkv=2, D=32, seed=0, q_zero=False):
    g = np.random.default_rng(seed)
    L = P + T
    lens = np.array([L], np.int32)
    bt, nb = W.block_table(g, lens)
    k = W.normal(g, (L, Hkv, D))
    v = W.normal(g, (L, Hkv, D))
    ks, vs = W.absmax_scales(k), W.absmax_scales(v)
    cache = Qn.cache_write(Qn.new_cache(nb, Hkv, D, "e4m3"), k, v, W.all_slots(bt, lens),
                           ks, vs, "e4m3")
    qf = np.zeros((T, Hq, D), np.float32) if q_zero else W.normal(g, (T, Hq, D))
    _, q = W.bf16_values(qf)
    qs = np.float32(max(np.abs(q).max(), 1e-30) / 448.0)
    return dict(q=q, cu=np.array([0, T], np.int32), cache=cache, bt=bt, lens=lens,
                qs=qs, ks=ks, vs=vs, T=T, P=P, D=D, Hkv=Hkv)


@pytest.mark.parametrize("window", [0, 9])
def test_mirror_without_p_quant_equals_exact(window):
    c = _prefill_case(T=50, P=20, seed=1)
    args = (c["q"], c["cu"], c["cache"], c["bt"], c["lens"], c["qs"], c["ks"], c["vs"],
            0.17, window)
    ex = A.prefill_exact(*args)
    for bn in (16, 64):
        mi = A.prefill_mirror(*args, kv_tile=bn, quantize_p=False)
        np.testing.assert_allclose(mi, ex, rtol=1e-12, atol=1e-14)


def test_prefill_uniform_scores_mean_of_visible_v():
    c = _prefill_case(T=37, P=11, seed=2, q_zero=True)
    got = A.prefill_mirror(c["q"], c["cu"], c["cache"], c["bt"], c["lens"], np.float32(1.0),
                           c["ks"], c["vs"], 0.3, 0, kv_tile=16)
    G = 2
    for i in range(c["T"]):
        pos = c["P"] + i
        for hq in range(4):
            h = hq // G
            vh = np.array([e4m3.decode(c["cache"][c["bt"][0][t // 16], h, 1, t % 16]) for t in range(pos + 1)])
            np.testing.assert_allclose(got[i, hq], vh.mean(axis=0) * c["vs"][h], rtol=1e-13)


def test_prefill_first_row_sees_only_key0():
    c = _prefill_case(T=20, P=0, seed=3)
    got = A.prefill_mirror(c["q"], c["cu"], c["cache"], c["bt"], c["lens"], c["qs"],
                           c["ks"], c["vs"], 0.2, 0, kv_tile=16, rows=[0])
    blk = c["bt"][0][0]
    for hq in range(4):
        h = hq // 2
        np.testing.assert_array_equal(got[0, hq], e4m3.decode(c["cache"][blk, h, 1, 0]) * np.float64(c["vs"][h]))


def test_prefill_rows_subset_matches_full():
    c = _prefill_case(T=45, P=30, seed=4)
    args = (c["q"], c["cu"], c["cache"], c["bt"], c["lens"], c["qs"], c["ks"], c["vs"], 0.2, 5)
    full = A.prefill_mirror(*args, kv_tile=16)
    rows = [0, 7, 44, 13]
    sub = A.prefill_mirror(*args, kv_tile=16, rows=rows)
    # BLAS may block the two products differently: equal up to fp64 rounding
    np.testing.assert_allclose(sub, full[rows], rtol=1e-13, atol=1e-15)


def test_prefill_literal_tiny():
    """Tiny causal prefill (T=6, P=3, D=4) by explicit loops against the
    mirror: scores from Q-hat and K-hat, tiles of 4, tile-running max."""
    c = _prefill_case(T=6, P=3, Hq=2, Hkv=1, D=4, seed=7)
    got = A.prefill_mirror(c["q"], c["cu"], c["cache"], c["bt"], c["lens"], c["qs"],
                           c["ks"], c["vs"], 0.5, 0, kv_tile=4)
    qcodes = [[[int(x) for x in e4m3.encode(np.array([np.float32(c["q"][i, hq, d]) / c["qs"]], dtype=np.float32))]
               for d in range(4)] for i in range(6) for hq in range(2)]
    for i in range(6):
        pos = 3 + i
        for hq in range(2):
            qh = [float(c["qs"]) * e4m3.decode_code(qcodes[i * 2 + hq][d][0]) for d in range(4)]
            s, vv, tiles = [], [], []
            for t in range(pos + 1):
                blk, r = int(c["bt"][0][t // 16]), t % 16
                kh = [float(c["ks"][0]) * e4m3.decode_code(int(c["cache"][blk, 0, 0, r, d])) for d in range(4)]
                vv.append([float(c["vs"][0]) * e4m3.decode_code(int(c["cache"][blk, 0, 1, r, d])) for d in range(4)])
                s.append(float(np.float32(0.5)) * sum(qh[d] * kh[d] for d in range(4)))
                tiles.append(t // 4)
            m, l, O = -math.inf, 0.0, [0.0] * 4
            for tile in sorted(set(tiles)):
                idx = [j for j in range(len(s)) if tiles[j] == tile]
                mn = max(m, max(s[j] for j in idx))
                a = 0.0 if m == -math.inf else math.exp(m - mn)
                acc, ls = [0.0] * 4, 0.0
                for j in idx:
                    p = math.exp(s[j] - mn)
                    pq = e4m3.decode_code(int(e4m3.encode(np.array([p]))[0]))
                    ls += p
                    for d in range(4):
                        acc[d] += pq * vv[j][d]
                O = [a * O[d] + acc[d] for d in range(4)]
                l = a * l + ls
                m = mn
            np.testing.assert_allclose(got[i, hq], [O[d] / l for d in range(4)], rtol=1e-12)


def test_flip_slack_covers_perturbed_scores():
    # scores perturbed by a relative 1e-7 (float32-sized error) may flip e4m3
    # roundings of p; the slack must bound the change of every output element
    g = np.random.default_rng(21)
    kv_tile = 16
    worst = 0.0
    for trial in range(200):
        n = int(g.integers(1, 60))
        keys = np.arange(n)
        s = g.standard_normal(n) * 2
        V = g.standard_normal((n, 4))
        o, slack = A.mirror_row(s, keys, V, kv_tile, True, 4e-6, True)
        for k in range(5):
            sp = s * (1 + g.uniform(-1e-7, 1e-7, n))
            op = A.mirror_row(sp, keys, V, kv_tile, True)
            excess = np.abs(op - o) - slack
            worst = max(worst, excess.max())
    # only float64 rounding noise (and the unquantised denominator's own
    # change, ~1e-7 relative) may remain
    assert worst < 1e-6, worst


def test_flip_slack_zero_without_midpoints():
    # p = 1 exactly and p = 0.5 exactly are codes, far from any midpoint
    s = np.array([0.0, np.log(0.5)])
    o, slack = A.mirror_row(s, np.arange(2), np.eye(2), 16, True, 4e-6, True)
    assert np.all(slack == 0)
