"""Helpers shared by the GPU parity tests: case builders and error metrics.

Inputs come from ``workloads`` (seeded); the GPU side fills its cache with the
library's own cache_write, the CPU side builds its cache with the oracle.
Nothing computed on the GPU is fed to the oracle.
"""

import math
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


def assert_gate(gpu, ref, what, max_abs=MAX_ABS, rel_l2=REL_L2):
    ma, rl = metrics(gpu, ref)
    log(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}"


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
                 q_zero=False):
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
            self.ks, self.vs = W.absmax_scales(k), W.absmax_scales(v)
        else:
            self.ks = self.vs = np.ones(Hkv, dtype=np.float32)
        self.slots = W.all_slots(self.bt, self.lens)
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
        self.cache = fa.new_cache(max(self.nblocks, 1), Hkv, D, cache_dtype)
        self.cache.view(torch.uint8).fill_(0)
        if N:
            fa.cache_write(dev(k), dev(v), dev(self.slots), dev(self.ks), dev(self.vs),
                           self.cache)
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
