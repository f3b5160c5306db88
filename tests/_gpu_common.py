"""Helpers shared by the GPU parity tests: case builders and error metrics.

Inputs come from ``workloads`` (seeded); the GPU side fills its cache with the
library's own cache_write, the CPU side builds its cache with the oracle.
Nothing computed on the GPU is fed to the oracle.
"""

import json
import math
import os
import sys

import numpy as np

import workloads as W
from oracle import quant as OQ

# Gate on attention outputs (max |gpu - oracle| and relative L2 over the
# whole output of a call).
MAX_ABS = 2e-3
REL_L2 = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def metrics(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = gpu - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def worst_row(gpu, ref):
    """(relative L2, index) of the output row (last axis) with the largest
    relative L2 error; rows whose reference is 0 count their absolute norm."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if gpu.size == 0:
        return 0.0, ()
    d = np.linalg.norm(gpu - ref, axis=-1)
    n = np.linalg.norm(ref, axis=-1)
    r = np.where(n > 0, d / np.where(n > 0, n, 1.0), d)
    i = np.unravel_index(int(np.argmax(r)), r.shape)
    return float(r[i]), tuple(int(x) for x in i)


def record(entry):
    """Append one parity result to the JSON-lines file named by
    FA8_PARITY_LOG (nothing when it is unset)."""
    path = os.environ.get("FA8_PARITY_LOG")
    if not path:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as f:
        f.write(json.dumps(entry) + "\n")


def assert_gate(gpu, ref, what, max_abs=MAX_ABS, rel_l2=REL_L2, slack=None, meta=None):
    """Gate: relative L2 of the raw difference, and max |gpu - ref| beyond
    ``slack`` (the oracle's per-element allowance for e4m3 roundings of p
    that a float32 kernel may legitimately take the other way; None = 0).
    ``meta`` (kernel, shape, context, mode, ...) goes into the parity record
    with the measured errors."""
    ma, rl = metrics(gpu, ref)
    diff = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    excess = diff if slack is None else np.maximum(diff - slack, 0.0)
    me = float(excess.max()) if excess.size else 0.0
    wr, wi = worst_row(gpu, ref)
    nref = float(np.linalg.norm(np.asarray(ref, np.float64)))
    rel_excess = float(np.linalg.norm(excess) / nref) if nref > 0 else float(np.linalg.norm(excess))
    extra = "" if slack is None else f" beyond-flip-allowance={me:.3e} (max allowance {float(np.max(slack)):.3e})"
    log(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e} worst_row_rel_l2={wr:.3e}{extra}")
    rec = dict(what=what, max_abs=ma, rel_l2=rl, excess=me, rel_l2_excess=rel_excess,
               worst_row_rel_l2=wr,
               worst_row=list(wi), elements=int(diff.size),
               finite=bool(np.all(np.isfinite(gpu))),
               passed=bool(me <= max_abs and rl <= rel_l2 and np.all(np.isfinite(gpu))))
    rec.update(meta or {})
    record(rec)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    assert me <= max_abs and rl <= rel_l2, f"{what}: max_abs={ma:.3e} excess={me:.3e} rel_l2={rl:.3e}"


def dev(x, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


class DecodeCase:
    """One decode layer: host inputs, the GPU cache (written by the GPU
    cache_write) and, on demand, the oracle cache of selected KV heads."""

    def __init__(self, B, Hq, Hkv, D, lens, cache_dtype="e4m3", seed=0,
                 outliers=False, scales="absmax", window=0, oracle_heads=None,
                 q_zero=False, fill=0, skip_last=False, window_only=False):
        import torch
        import attention_fp8_quantized_amd as fa
        self.B, self.Hq, self.Hkv, self.D = B, Hq, Hkv, D
        self.lens = np.asarray(lens, dtype=np.int32)
        self.cd, self.window = cache_dtype, window
        g = np.random.default_rng(seed)
        self.bt, self.nblocks = W.block_table(g, self.lens)
        N = int(self.lens.sum())
        gk = W.rng(seed, 0, W.K)
        gv = W.rng(seed, 0, W.V)
        k = W.normal(gk, (N, Hkv, D))
        v = W.normal(gv, (N, Hkv, D))
        if outliers:
            k = W.with_outliers(k, W.rng(seed, 0, W.OUTLIERS))
            v = W.with_outliers(v, W.rng(seed, 1, W.OUTLIERS))
        if scales == "absmax" and N:
            fm = W.FMT_MAX.get(cache_dtype, W.E4M3_MAX)
            self.ks, self.vs = W.absmax_scales(k, fm), W.absmax_scales(v, fm)
        else:
            self.ks = self.vs = np.ones(Hkv, dtype=np.float32)
        self.slots = W.all_slots(self.bt, self.lens)
        # window_only: only the keys the window shows are written, and the
        # table entries of pages wholly before the window name one extra
        # block that is never written (it keeps the fill bytes, NaN codes
        # with fill=0xFF): nothing outside the window may reach the output
        self.visible = np.ones(N, dtype=bool)
        if window_only:
            assert window > 0
            sentinel = self.nblocks
            self.nblocks += 1
            at = 0
            for b, L in enumerate(self.lens):
                lo = max(0, int(L) - window)
                self.visible[at:at + lo] = False
                self.bt[b, :lo // 16] = sentinel
                at += int(L)
        # host-side bounds checks before anything is launched
        need = W.blocks_needed(self.lens)
        for b, n in enumerate(need):
            assert np.all((self.bt[b, :n] >= 0) & (self.bt[b, :n] < max(self.nblocks, 1)))
        assert self.bt.shape[1] * 16 >= (int(self.lens.max()) if B else 0)
        assert len(self.slots) == N and (N == 0 or self.slots.max() < self.nblocks * 16)
        qb, self.q = W.bf16_values(np.zeros((B, Hq, D), np.float32) if q_zero
                                   else W.normal(W.rng(seed, 0, W.Q), (B, Hq, D)))
        self.k, self.v = k, v
        # GPU side
        # cache bytes before the writes: rows past each sequence end keep
        # them (0xFF is a NaN code in e4m3 and a NaN half-word in bf16)
        self.cache = fa.new_cache(max(self.nblocks, 1), Hkv, D, cache_dtype)
        self.cache.view(torch.uint8).fill_(fill)
        # skip_last: each sequence's last token stays unwritten (the current
        # decode token, to be appended by the caller)
        ends = np.cumsum(self.lens) - 1
        self.last_idx = ends[self.lens > 0]
        write = self.visible.copy()
        if skip_last:
            write[self.last_idx] = False
        if write.any():
            fa.cache_write(dev(k[write]), dev(v[write]), dev(self.slots[write]), dev(self.ks),
                           dev(self.vs), self.cache)
        self.q_dev = qb.cuda()
        self.bt_dev = dev(self.bt)
        self.lens_dev = dev(self.lens)
        self.ks_dev, self.vs_dev = dev(self.ks), dev(self.vs)
        self.sm = np.float32(1.0 / math.sqrt(D))
        self.oracle_heads = list(range(Hkv)) if oracle_heads is None else list(oracle_heads)

    def run_gpu(self, num_splits=0, **kw):
        import torch
        import attention_fp8_quantized_amd as fa
        out = fa.decode_attention(self.q_dev, self.cache, self.bt_dev, self.lens_dev,
                                  self.ks_dev, self.vs_dev, float(self.sm),
                                  int(self.lens.max()) if self.B else 0,
                                  window=self.window, num_splits=num_splits, **kw)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle(self):
        """Oracle output restricted to the query heads of ``oracle_heads``
        (returns (out [B][len(heads)*G][D], list of query-head indices))."""
        from oracle import attention as OA
        G = self.Hq // self.Hkv
        outs, qheads = [], []
        for h in self.oracle_heads:
            # the oracle cache holds only this KV head (and only rows the
            # window can see); every row comes from the host inputs
            cache = OQ.new_cache(max(self.nblocks, 1), 1, self.D, self.cd)
            keep = np.ones(len(self.slots), dtype=bool)
            if self.window > 0:
                keep[:] = False
                at = 0
                for L in self.lens:
                    lo = max(0, int(L) - self.window)
                    keep[at + lo:at + int(L)] = True
                    at += int(L)
            OQ.cache_write(cache, self.k[keep][:, h:h + 1], self.v[keep][:, h:h + 1],
                           self.slots[keep], self.ks[h:h + 1], self.vs[h:h + 1], self.cd)
            q = self.q[:, h * G:(h + 1) * G, :]
            o = OA.decode_attention(q, cache, self.bt, self.lens, self.ks[h:h + 1],
                                    self.vs[h:h + 1], self.sm, self.window, self.cd, 1)
            outs.append(o)
            qheads += list(range(h * G, (h + 1) * G))
        return np.concatenate(outs, axis=1), qheads


class PrefillCase:
    """Chunked prefill over a paged FP8 cache (e4m3 or e5m2 codes): sequence
    b has context lens[b] whose last qlens[b] tokens are the queries (packed
    by cu)."""

    def __init__(self, qlens, lens, Hq, Hkv, D, seed=0, window=0, q_zero=False,
                 q_scale="absmax", fill=0, cache_dtype="e4m3", window_only=False):
        import torch
        import attention_fp8_quantized_amd as fa
        self.qlens = np.asarray(qlens, dtype=np.int32)
        self.lens = np.asarray(lens, dtype=np.int32)
        assert np.all(self.lens >= self.qlens)
        self.B = len(self.lens)
        self.Hq, self.Hkv, self.D, self.window = Hq, Hkv, D, window
        g = np.random.default_rng(seed)
        self.bt, self.nblocks = W.block_table(g, self.lens)
        N = int(self.lens.sum())
        k = W.normal(W.rng(seed, 0, W.K), (N, Hkv, D))
        v = W.normal(W.rng(seed, 0, W.V), (N, Hkv, D))
        self.cd = cache_dtype
        fm = W.FMT_MAX[cache_dtype]
        self.ks, self.vs = W.absmax_scales(k, fm), W.absmax_scales(v, fm)
        self.slots = W.all_slots(self.bt, self.lens)
        # window_only: only keys some query of the chunk can see are written
        # (from the first query's window start on); the table entries of
        # pages wholly before it name one extra block that is never written
        self.write = np.ones(N, dtype=bool)
        if window_only:
            assert window > 0
            sentinel = self.nblocks
            self.nblocks += 1
            at = 0
            for b, (L, T) in enumerate(zip(self.lens, self.qlens)):
                lo = max(0, int(L) - int(T) - window + 1)
                self.write[at:at + lo] = False
                self.bt[b, :lo // 16] = sentinel
                at += int(L)
        need = W.blocks_needed(self.lens)
        for b, nb in enumerate(need):
            assert np.all((self.bt[b, :nb] >= 0) & (self.bt[b, :nb] < self.nblocks))
        assert self.slots.max() < self.nblocks * 16
        self.cu = np.concatenate([[0], np.cumsum(self.qlens)]).astype(np.int32)
        Tq = int(self.cu[-1])
        qf = np.zeros((Tq, Hq, D), np.float32) if q_zero else W.normal(W.rng(seed, 0, W.Q), (Tq, Hq, D))
        qb, self.q = W.bf16_values(qf)
        if q_scale == "absmax":
            self.qs = np.array([max(float(np.abs(self.q).max()), 1e-30) / 448.0], np.float32)
        else:
            self.qs = np.array([q_scale], np.float32)
        self.k, self.v = k, v
        self.cache = fa.new_cache(self.nblocks, Hkv, D, cache_dtype)
        self.cache.view(torch.uint8).fill_(fill)
        w = self.write
        fa.cache_write(dev(k[w]), dev(v[w]), dev(self.slots[w]), dev(self.ks), dev(self.vs),
                       self.cache)
        self.q_dev = qb.cuda()
        self.dev = {n: dev(a) for n, a in dict(cu=self.cu, bt=self.bt, lens=self.lens,
                                                qs=self.qs, ks=self.ks, vs=self.vs).items()}
        self.sm = np.float32(1.0 / math.sqrt(D))
        self._oracle_cache = None

    def run_gpu(self, accum_mode=1):
        import torch
        import attention_fp8_quantized_amd as fa
        d = self.dev
        out = fa.prefill_attention(self.q_dev, d["cu"], self.cache, d["bt"], d["lens"], d["qs"],
                                   d["ks"], d["vs"], float(self.sm), int(self.qlens.max()),
                                   window=self.window, accum_mode=accum_mode)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle_cache(self):
        if self._oracle_cache is None:
            c = OQ.new_cache(self.nblocks, self.Hkv, self.D, self.cd)
            w = self.write
            self._oracle_cache = OQ.cache_write(c, self.k[w], self.v[w], self.slots[w], self.ks,
                                                self.vs, self.cd)
        return self._oracle_cache

    # float32 score and exp2 error of the kernel, relative, with a 4x margin
    FLIP_TOL = 4e-6

    def oracle(self, rows=None, exact=False):
        """(reference, flip allowance) for the mirror; the reference alone
        for the unquantised-P reference (exact=True)."""
        import attention_fp8_quantized_amd as fa
        from oracle import attention as OA
        args = (self.q, self.cu, self.oracle_cache(), self.bt, self.lens, self.qs[0], self.ks,
                self.vs, self.sm, self.window)
        if exact:
            return OA.prefill_exact(*args, rows=rows, cache_dtype=self.cd)
        return OA.prefill_mirror(*args, kv_tile=fa.prefill_kv_tile(self.D), rows=rows,
                                 flip_tol=self.FLIP_TOL, cache_dtype=self.cd)
