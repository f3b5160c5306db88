"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds no part of the method's arithmetic: it draws random
numbers, lays out block tables and slot ids, and picks per-head scales the
way a calibration stand-in would (absmax / 448).  The quantisation, the cache
write and the attention itself live on each side separately (``oracle/`` on
the CPU, the HIP library on the GPU).

Seeds follow one rule so that every input can be regenerated:
    seed = 1000 * config + 10 * layer + tensor
with tensor 0 = Q, 1 = K, 2 = V, 3 = outlier channels, 4 = block permutation,
5 = sequence lengths.

Workload shapes stand in for the pages' models ([BLOG] "Performance
benchmarks"): a Llama-3.1-8B-shaped layer (32 query / 8 KV heads, head_dim
128), a gpt-oss-20b-shaped hybrid stack (64 / 8, head_dim 64, window 128) and
a head_dim-256 model (8 / 1).  No model weights or datasets are involved.
"""

import math

import numpy as np

BLOCK_SIZE = 16
E4M3_MAX = 448.0
E5M2_MAX = 57344.0
FMT_MAX = {"e4m3": E4M3_MAX, "e5m2": E5M2_MAX}

Q, K, V, OUTLIERS, BLOCKS, LENGTHS = range(6)


def rng(config, layer, tensor):
    return np.random.default_rng(1000 * config + 10 * layer + tensor)


def normal(gen, shape):
    """float32 N(0, 1) draws."""
    return gen.standard_normal(shape, dtype=np.float32)


def with_outliers(x, gen, fraction=0.01, factor=20.0):
    """Multiply round(fraction * H * D) distinct (head, channel) pairs of
    x[N][H][D] by ``factor`` (the "1% outlier channels x20" recipe)."""
    _, H, D = x.shape
    n = int(round(fraction * H * D))
    pick = gen.choice(H * D, size=n, replace=False)
    x = x.copy()
    for p in pick:
        x[:, p // D, p % D] *= np.float32(factor)
    return x


def absmax_scales(x, fmt_max=E4M3_MAX):
    """Per-head scale fl32(max |x[:, h, :]|) / fmt_max (float32 [H]; fmt_max
    448 for an e4m3 cache, 57344 for e5m2); 1.0 for an all-zero head."""
    a = np.abs(np.asarray(x, dtype=np.float32)).max(axis=(0, 2))
    s = (a / np.float32(fmt_max)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    return s


def bf16_values(x):
    """Round float32 draws to bfloat16 the way the inputs are produced (by
    torch's cast), returned both as a torch bf16 tensor and as the exact
    float32 values for the CPU side."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t, t.to(torch.float32).numpy()


def blocks_needed(seq_lens):
    return [int(math.ceil(int(L) / BLOCK_SIZE)) for L in seq_lens]


def block_table(gen, seq_lens, pool_factor=1.25, min_blocks_per_seq=None):
    """Block table int32 [B][max_blocks] whose entries are a seeded
    permutation of a pool ``pool_factor`` times larger than needed, so that
    logical pages never sit in physical order.  Unused entries are -1."""
    need = blocks_needed(seq_lens)
    total = sum(need)
    pool = max(int(math.ceil(total * pool_factor)), total, 1)
    perm = gen.permutation(pool).astype(np.int32)
    width = max(max(need) if need else 0, min_blocks_per_seq or 0, 1)
    bt = np.full((len(seq_lens), width), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[at:at + n]
        at += n
    return bt, pool


def slots(bt, b, lo, hi):
    """Slot ids (int64) of tokens lo..hi-1 of sequence b."""
    t = np.arange(lo, hi, dtype=np.int64)
    return bt[b, t // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + t % BLOCK_SIZE


def all_slots(bt, seq_lens):
    """Slot ids of every token of every sequence, sequences concatenated."""
    return np.concatenate([slots(bt, b, 0, int(L)) for b, L in enumerate(seq_lens)]) \
        if len(seq_lens) else np.zeros(0, dtype=np.int64)


def uniform_lengths(gen, batch, lo, hi):
    """Sequence lengths drawn uniformly from the integers lo..hi."""
    return gen.integers(lo, hi + 1, size=batch).astype(np.int32)


# Workload shapes (the five configurations the bench and the tests use)
CONFIGS = {
    1: dict(name="single-layer fp8 decode, hd64 GQA4, ctx 512",
            B=1, Hq=8, Hkv=2, D=64, contexts=[512], window=0),
    2: dict(name="Llama-3.1-8B-shaped decode layer, hd128 GQA4",
            B=1, Hq=32, Hkv=8, D=128, contexts=[1024, 8192, 32768, 131072],
            window=0),
    3: dict(name="loaded decode, 8 seqs x U{18000..22000}, 32 layers",
            B=8, Hq=32, Hkv=8, D=128, len_lo=18000, len_hi=22000, layers=32,
            window=0),
    4: dict(name="gpt-oss-20b-shaped hybrid, 24 layers (12 full fp8 + 12 SW-128 bf16)",
            B=8, Hq=64, Hkv=8, D=64, context=20000, layers=24, window_sw=128),
    5: dict(name="hd256 fp8 prefill 32k + decode 128k, 8/1 heads",
            B=1, Hq=8, Hkv=1, D=256, prefill_T=32768, decode_ctx=131072),
}
