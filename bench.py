"""Benchmark: FP8 paged-KV decode on one MI355X.

Workload (one step): a Llama-3.1-8B-shaped decode step over 32 independent
layers -- 32 query / 8 KV heads, head_dim 128, block size 16, batch 1,
32k-token context, K/V ~ N(0,1) with 1% outlier channels x20 and per-KV-head
absmax/448 scales.  Per layer the step writes the current token's K/V into
the FP8 cache (cache_write) and runs decode attention over the whole context.
The 32 layer caches (2.1 GB) are distinct so the 256 MB last-level cache
cannot serve repeated reads.

Printed: one JSON line with
  value      algorithmic KV GB/s of the whole step (decode + cache write)
  roofline   the decode kernel alone, timed with HIP events on its stream,
             against the 8 TB/s HBM peak
  slope      decode time per context token for the FP8 and the BF16 cache
             (same kernel), fitted over contexts {1k, 8k, 32k, 128k} as
             t = slope * ctx + intercept, and their ratio
  prefill    (when built) head_dim-256 FP8 prefill chunk throughput vs the
             5 PFLOP/s dense FP8 MFMA peak
  cpu_baseline  the fp64 NumPy oracle decoding one layer of the same
             workload on the host cores

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick]
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, TFLOP/s


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------

def decode_bytes(B, Hq, Hkv, D, ctx, elem):
    """Bytes decode must move: K and V of every visible token, q in (bf16),
    out (fp32), the block-table entries and the two scale vectors."""
    n = ctx
    kv = B * n * Hkv * D * 2 * elem
    qo = B * Hq * D * (2 + 4)
    bt = B * math.ceil(n / 16) * 4
    sc = 8 * Hkv
    return kv + qo + bt + sc


def cache_write_bytes(N, Hkv, D, in_bytes, elem):
    return N * Hkv * D * 2 * (in_bytes + elem)


# ---------------------------------------------------------------------------
# synthetic caches on the device
# ---------------------------------------------------------------------------

def fill_pool(fa, torch, pool_blocks, Hkv, D, cache_dtype, seed, outliers=True):
    """A pool of blocks filled through the library's cache_write from
    N(0,1) K/V (seeded device RNG) with 1% outlier channels x20 and
    absmax/448 per-head scales.  Returns (cache, k_scale, v_scale)."""
    dev = torch.device("cuda")
    cache = fa.new_cache(pool_blocks, Hkv, D, cache_dtype, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    n_out = int(round(0.01 * Hkv * D))
    pick_k = torch.randperm(Hkv * D, generator=gen, device=dev)[:n_out]
    pick_v = torch.randperm(Hkv * D, generator=gen, device=dev)[:n_out]
    mul_k = torch.ones(Hkv * D, device=dev)
    mul_k[pick_k] = 20.0
    mul_v = torch.ones(Hkv * D, device=dev)
    mul_v[pick_v] = 20.0
    mul_k, mul_v = mul_k.view(1, Hkv, D), mul_v.view(1, Hkv, D)
    # scales: absmax over the whole pool's draws; N(0,1) absmax over this
    # many draws is ~5.5-6, x20 outliers dominate: use the outlier-aware max
    total = pool_blocks * 16
    chunk = 1 << 16
    amax_k = torch.zeros(Hkv, device=dev)
    amax_v = torch.zeros(Hkv, device=dev)
    state = gen.get_state()
    for t0 in range(0, total, chunk):
        n = min(chunk, total - t0)
        k = torch.randn((n, Hkv, D), generator=gen, device=dev) * mul_k
        v = torch.randn((n, Hkv, D), generator=gen, device=dev) * mul_v
        amax_k = torch.maximum(amax_k, k.abs().amax(dim=(0, 2)))
        amax_v = torch.maximum(amax_v, v.abs().amax(dim=(0, 2)))
    ks = (amax_k / 448.0).float().contiguous()
    vs = (amax_v / 448.0).float().contiguous()
    gen.set_state(state)
    for t0 in range(0, total, chunk):
        n = min(chunk, total - t0)
        k = torch.randn((n, Hkv, D), generator=gen, device=dev) * mul_k
        v = torch.randn((n, Hkv, D), generator=gen, device=dev) * mul_v
        slots = torch.arange(t0, t0 + n, device=dev, dtype=torch.int64)
        fa.cache_write(k.contiguous(), v.contiguous(), slots, ks, vs, cache)
    torch.cuda.synchronize()
    return cache, ks, vs


def layer_tables(torch, layers, blocks_per_layer, pool_blocks, seed):
    """int32 [layers][blocks_per_layer]: each layer owns distinct pool blocks
    (a seeded permutation, so logical pages are never in physical order)."""
    g = torch.Generator()
    g.manual_seed(seed)
    need = layers * blocks_per_layer
    assert need <= pool_blocks
    perm = torch.randperm(pool_blocks, generator=g)[:need].to(torch.int32)
    return perm.view(layers, blocks_per_layer).cuda()


# ---------------------------------------------------------------------------
# measurements
# ---------------------------------------------------------------------------

def time_decode(fa, torch, cache, tables, ks, vs, q, ctx, D, reps, splits=0):
    """Average time (ms) of one decode call, cycling through the layers'
    block tables; HIP events on the stream the kernel is launched on."""
    B = q.shape[0]
    lens = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    layers = tables.shape[0]
    S = splits or fa.decode_num_splits(B, cache.shape[1], ctx)
    ws = fa.new_decode_workspace(fa.decode_workspace_bytes(B, q.shape[1], D, S))
    out = torch.empty((B, q.shape[1], D), dtype=torch.float32, device="cuda")
    sm = 1.0 / math.sqrt(D)
    bts = [tables[i:i + 1].expand(B, -1).contiguous() for i in range(layers)]
    for i in range(min(layers, 4)):      # warm-up
        fa.decode_attention(q, cache, bts[i], lens, ks, vs, sm, ctx, num_splits=S,
                            out=out, workspace=ws)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    n = 0
    for _ in range(reps):
        for i in range(layers):
            fa.decode_attention(q, cache, bts[i], lens, ks, vs, sm, ctx, num_splits=S,
                                out=out, workspace=ws)
            n += 1
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n, S


def slope_fit(ctxs, times):
    A = np.vstack([np.asarray(ctxs, float), np.ones(len(ctxs))]).T
    (slope, icpt), *_ = np.linalg.lstsq(A, np.asarray(times, float), rcond=None)
    return float(slope), float(icpt)


def measure_slope(fa, torch, Hq, Hkv, D, contexts, min_pool_bytes, reps):
    """Per-layer decode time at each context for the FP8 and the BF16 cache
    (same kernel), over enough distinct layers that the working set exceeds
    the last-level cache.  Returns dict with times, slopes and ratio."""
    res = {}
    q = torch.randn((1, Hq, D), device="cuda").to(torch.bfloat16)
    for cd, elem in (("e4m3", 1), ("bf16", 2)):
        blocks_max = math.ceil(max(contexts) / 16)
        page_bytes = 2 * Hkv * 16 * D * elem
        pool = max(math.ceil(min_pool_bytes / page_bytes), 4 * blocks_max)
        cache, ks, vs = fill_pool(fa, torch, pool, Hkv, D, cd, seed=2000 + elem)
        times = []
        for ctx in contexts:
            bpl = math.ceil(ctx / 16)
            layers = max(1, min(pool // bpl, 256))
            tables = layer_tables(torch, layers, bpl, pool, seed=ctx)
            t, S = time_decode(fa, torch, cache, tables, ks, vs, q, ctx, D,
                               reps=max(1, reps * 32 // layers))
            times.append(t)
            log(f"  slope point {cd} ctx={ctx}: {t * 1e3:.2f} us/layer "
                f"({decode_bytes(1, Hq, Hkv, D, ctx, elem) / t / 1e6:.0f} GB/s, S={S}, "
                f"{layers} layers)")
        s, i = slope_fit(contexts, times)
        res[cd] = dict(ms_per_layer=times, slope_ms_per_token=s, intercept_ms=i)
        del cache
        torch.cuda.empty_cache()
    res["ratio_fp8_over_bf16"] = res["e4m3"]["slope_ms_per_token"] / res["bf16"]["slope_ms_per_token"]
    s8, i8 = res["e4m3"]["slope_ms_per_token"], res["e4m3"]["intercept_ms"]
    s16, i16 = res["bf16"]["slope_ms_per_token"], res["bf16"]["intercept_ms"]
    res["break_even_tokens"] = (i8 - i16) / (s16 - s8) if s16 != s8 else None
    res["contexts"] = list(contexts)
    return res


def cpu_baseline(Hq, Hkv, D, ctx, budget_s=10.0):
    """The fp64 oracle decoding one Llama-shaped layer at ``ctx`` on the host
    (bounded sample: one layer, repeated until ``budget_s`` of CPU time)."""
    import workloads as W
    from oracle import attention as OA
    from oracle import quant as OQ
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    lens = np.array([ctx], np.int32)
    bt, nb = W.block_table(W.rng(2, 0, W.BLOCKS), lens)
    k = W.with_outliers(W.normal(W.rng(2, 0, W.K), (ctx, Hkv, D)), W.rng(2, 0, W.OUTLIERS))
    v = W.with_outliers(W.normal(W.rng(2, 0, W.V), (ctx, Hkv, D)), W.rng(2, 1, W.OUTLIERS))
    ks, vs = W.absmax_scales(k), W.absmax_scales(v)
    cache = OQ.cache_write(OQ.new_cache(nb, Hkv, D, "e4m3"), k, v, W.all_slots(bt, lens),
                           ks, vs, "e4m3")
    del k, v
    _, q = W.bf16_values(W.normal(W.rng(2, 0, W.Q), (1, Hq, D)))
    sm = np.float32(1 / math.sqrt(D))
    n = 0
    t0 = time.perf_counter()
    while True:
        OA.decode_attention(q, cache, bt, lens, ks, vs, sm, 0, "e4m3", Hkv)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per_layer = el / n
    gbs = decode_bytes(1, Hq, Hkv, D, ctx, 1) / per_layer / 1e9
    cores = len(os.sched_getaffinity(0))
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": min(cores, max(blas_threads, 1)),
            "kind": "oracle",
            "sample": f"{n} decode call(s) of one {ctx}-token Llama-shaped layer "
                      f"(32/8 heads, hd128, fp8 cache), fp64 NumPy, "
                      f"{per_layer * 1e3:.1f} ms per layer; host cores available {cores}, "
                      f"BLAS threads {blas_threads}"}


def measure_prefill(fa, torch, T=32768, Hq=8, Hkv=1, D=256, reps=3, accum_mode=1):
    """Causal prefill chunk of T tokens (P = 0) on the head_dim-256 shape."""
    dev = torch.device("cuda")
    nb = math.ceil(T / 16)
    cache, ks, vs = fill_pool(fa, torch, nb, Hkv, D, "e4m3", seed=5000, outliers=False)
    bt = torch.randperm(nb, generator=torch.Generator().manual_seed(5)).to(torch.int32)
    bt = bt.view(1, nb).cuda()
    q = torch.randn((T, Hq, D), device=dev).to(torch.bfloat16)
    qs = (q.float().abs().amax() / 448.0).view(1).contiguous()
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    lens = torch.tensor([T], dtype=torch.int32, device=dev)
    out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    sm = 1.0 / math.sqrt(D)
    fa.prefill_attention(q, cu, cache, bt, lens, qs, ks, vs, sm, T, accum_mode=accum_mode,
                         out=out)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fa.prefill_attention(q, cu, cache, bt, lens, qs, ks, vs, sm, T,
                             accum_mode=accum_mode, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    pairs = T * (T + 1) / 2
    flops = 4.0 * D * Hq * pairs
    return {"T": T, "heads": f"{Hq}/{Hkv}", "head_dim": D, "accum_mode": accum_mode,
            "ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 2),
            "frac_fp8_peak": round(flops / ms / 1e9 / FP8_MFMA_PEAK_TFLOPS, 4)}


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--ctx", type=int, default=32768)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--quick", action="store_true", help="skip slope, prefill and CPU legs")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-slope", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_fp8_quantized_amd as fa
    fa.load()
    torch.cuda.init()

    B, Hq, Hkv, D, ctx, layers = 1, 32, 8, 128, args.ctx, args.layers
    bpl = math.ceil(ctx / 16)
    pool = bpl * layers
    log(f"filling {layers} FP8 layers x {ctx} tokens ({pool * 2 * Hkv * 16 * D / 1e9:.2f} GB)")
    cache, ks, vs = fill_pool(fa, torch, pool, Hkv, D, "e4m3", seed=1000)
    tables = layer_tables(torch, layers, bpl, pool, seed=1)
    dev = torch.device("cuda")
    gq = torch.Generator(device=dev)
    gq.manual_seed(3)
    qs = [torch.randn((B, Hq, D), generator=gq, device=dev).to(torch.bfloat16)
          for _ in range(layers)]
    knew = [torch.randn((B, Hkv, D), generator=gq, device=dev) for _ in range(layers)]
    vnew = [torch.randn((B, Hkv, D), generator=gq, device=dev) for _ in range(layers)]
    lens = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    bts = [tables[i:i + 1].contiguous() for i in range(layers)]
    # the current token (position ctx-1) of each layer
    slot_new = [(tables[i, (ctx - 1) // 16].to(torch.int64) * 16 + (ctx - 1) % 16).view(1)
                for i in range(layers)]
    S = args.splits or fa.decode_num_splits(B, Hkv, ctx)
    ws = fa.new_decode_workspace(fa.decode_workspace_bytes(B, Hq, D, S))
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    sm = 1.0 / math.sqrt(D)

    def step():
        for i in range(layers):
            fa.cache_write(knew[i], vnew[i], slot_new[i], ks, vs, cache)
            fa.decode_attention(qs[i], cache, bts[i], lens, ks, vs, sm, ctx, num_splits=S,
                                out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"step: {ms_step:.4f} ms (events), wall {wall / args.steps * 1e3:.4f} ms")

    step_bytes = layers * (decode_bytes(B, Hq, Hkv, D, ctx, 1) +
                           cache_write_bytes(B, Hkv, D, 4, 1))
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # dominant kernel alone: the decode launch (one kernel per call)
    dec_ms, _ = time_decode(fa, torch, cache, tables, ks, vs, qs[0], ctx, D,
                            reps=max(args.steps, 5), splits=S)
    per_launch = decode_bytes(B, Hq, Hkv, D, ctx, 1)
    achieved = per_launch / (dec_ms * 1e-3) / 1e9
    log(f"decode kernel: {dec_ms * 1e3:.2f} us/launch -> {achieved:.0f} GB/s "
        f"({achieved / HBM_PEAK_GBS * 100:.1f}% of peak), splits={S}")
    del cache
    torch.cuda.empty_cache()

    result = {
        "metric": "FP8 decode KV GB/s (% of HBM peak) + ms/ctx-token slope vs BF16 cache",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 cache, f32 math",
        "data": "synthetic: N(0,1) K/V with 1% outlier channels x20, absmax/448 per-KV-head "
                "scales, device RNG",
        "config": {"workload": "Llama-3.1-8B-shaped FP8 decode layer x32 distinct layers",
                   "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "block_size": 16, "context": ctx, "layers": layers, "splits": S},
        "pct_hbm_peak": round(value / HBM_PEAK_GBS * 100, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": f"decode_split_kernel<128,4,fp8,4> ({per_launch} algorithmic "
                               f"bytes/launch, {dec_ms * 1e3:.3f} us avg over "
                               f"{max(args.steps, 5) * layers} launches)"},
    }
    if not args.quick and not args.no_slope:
        log("slope: FP8 vs BF16 cache, same kernel")
        result["slope"] = measure_slope(fa, torch, Hq, Hkv, D, [1024, 8192, 32768, 131072],
                                        min_pool_bytes=1.1e9, reps=3)
    if not args.quick and not args.no_prefill:
        try:
            result["prefill"] = [measure_prefill(fa, torch, accum_mode=1),
                                 measure_prefill(fa, torch, accum_mode=0)]
        except fa.Fa8Error as e:
            result["prefill"] = f"not measured: {e}"
    if not args.quick and not args.no_cpu:
        log("cpu baseline: oracle decode")
        result["cpu_baseline"] = cpu_baseline(Hq, Hkv, D, ctx)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
