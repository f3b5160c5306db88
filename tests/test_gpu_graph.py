"""Every entry point captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: per-head scales, cache write, causal prefill, fused append + decode
(one merger per set) and plain decode (96 splits: the merge shared by the
last arrivals of the split groups).

The calls take their scales, lengths and inputs from device memory and
allocate nothing, so a captured call replays with whatever those buffers hold.
The test replays one graph over several decode steps.  Between replays it
rewrites the inputs and grows the decode lengths with eager work.  Every
replay must equal an eager run of the same calls on the same inputs bit for
bit: outputs, scales and cache bytes.  The eager path is the one the parity
tests check against the oracle.
"""

import math

import numpy as np
import pytest

import workloads as W
from _gpu_common import dev, log

pytestmark = pytest.mark.gpu

B, HQ, HKV, D = 3, 32, 8, 128
STEPS = 4
BASE = [700, 1500, 2100]      # decode contexts before the first step
P_LEN, P_Q = 1536, 512        # prefill sequence and its query chunk
TWO_LEVEL_SPLITS = 96         # > 64 splits: group counters, merge shared by slices


class Path:
    """Caches, scales, outputs and workspaces of one copy of the path."""

    def __init__(self, torch, fa, cache_d, cache_p, splits_a):
        self.cache_d = cache_d.clone()
        self.cache_p = cache_p.clone()
        self.ks_p = torch.zeros(HKV, dtype=torch.float32, device="cuda")
        self.vs_p = torch.zeros_like(self.ks_p)
        self.out_p = torch.zeros((P_Q, HQ, D), dtype=torch.float32, device="cuda")
        self.out_a = torch.zeros((B, HQ, D), dtype=torch.float32, device="cuda")
        self.out_d = torch.zeros_like(self.out_a)
        self.ws_a = fa.new_decode_workspace(fa.decode_workspace_bytes(B, HQ, D, splits_a))
        self.ws_d = fa.new_decode_workspace(fa.decode_workspace_bytes(B, HQ, D, TWO_LEVEL_SPLITS))

    def state(self):
        return [self.out_p, self.out_a, self.out_d, self.ks_p, self.vs_p, self.cache_d,
                self.cache_p]


def _run(fa, x, s):
    """One pass of the whole path on copy ``s`` with the inputs ``x``."""
    fa.absmax_scales(x["kp"], x["vp"], s.ks_p, s.vs_p)
    fa.cache_write(x["kp"], x["vp"], x["slots_p"], s.ks_p, s.vs_p, s.cache_p)
    fa.prefill_attention(x["qp"], x["cu"], s.cache_p, x["bt_p"], x["lens_p"], x["qs"],
                         s.ks_p, s.vs_p, x["sm"], P_Q, out=s.out_p)
    fa.decode_attention_append(x["q"], x["k_new"], x["v_new"], s.cache_d, x["bt_d"],
                               x["lens_d"], x["ks_d"], x["vs_d"], x["sm"], x["max_len"],
                               num_splits=x["splits_a"], out=s.out_a, workspace=s.ws_a)
    fa.decode_attention(x["q"], s.cache_d, x["bt_d"], x["lens_d"], x["ks_d"], x["vs_d"],
                        x["sm"], x["max_len"], num_splits=TWO_LEVEL_SPLITS, out=s.out_d,
                        workspace=s.ws_d)


def _bits(t):
    import torch
    return t.contiguous().view(torch.uint8).cpu().numpy()


def _refresh(torch, x, gen):
    """New step inputs, written in place into the captured buffers."""
    for name in ("kp", "vp", "k_new", "v_new"):
        x[name].copy_(torch.randn(x[name].shape, generator=gen, device="cuda"))
    x["qp"].copy_(torch.randn(x["qp"].shape, generator=gen, device="cuda").to(torch.bfloat16))
    x["q"].copy_(torch.randn(x["q"].shape, generator=gen, device="cuda").to(torch.bfloat16))
    x["qs"].copy_(x["qp"].float().abs().amax().reshape(1) / 448.0)


def test_graph_replays_match_eager():
    import torch
    import attention_fp8_quantized_amd as fa
    fa.load()
    max_len = max(BASE) + STEPS
    splits_a = fa.decode_num_splits(B, HKV, max_len)
    assert splits_a <= 64 < TWO_LEVEL_SPLITS
    g = np.random.default_rng(23)

    # decode: sequences sized for every step's appended token
    final = np.asarray(BASE, np.int32) + STEPS
    bt_d, nb_d = W.block_table(g, final)
    n0 = int(np.sum(BASE))
    k0 = W.normal(W.rng(23, 0, W.K), (n0, HKV, D))
    v0 = W.normal(W.rng(23, 0, W.V), (n0, HKV, D))
    ks_d, vs_d = W.absmax_scales(k0), W.absmax_scales(v0)
    slots0 = W.all_slots(bt_d, np.asarray(BASE, np.int32))
    assert slots0.max() < nb_d * 16 and bt_d.shape[1] * 16 >= int(final.max())
    cache_d = fa.new_cache(nb_d, HKV, D, "e4m3")
    cache_d.view(torch.uint8).fill_(0)
    fa.cache_write(dev(k0), dev(v0), dev(slots0), dev(ks_d), dev(vs_d), cache_d)

    # prefill: one sequence of P_LEN tokens, the last P_Q of them queries
    bt_p, nb_p = W.block_table(g, [P_LEN])
    slots_p = W.all_slots(bt_p, [P_LEN])
    assert slots_p.max() < nb_p * 16
    cache_p = fa.new_cache(nb_p, HKV, D, "e4m3")
    cache_p.view(torch.uint8).fill_(0)

    x = dict(
        kp=torch.zeros((P_LEN, HKV, D), device="cuda"),
        vp=torch.zeros((P_LEN, HKV, D), device="cuda"),
        qp=torch.zeros((P_Q, HQ, D), dtype=torch.bfloat16, device="cuda"),
        qs=torch.ones(1, device="cuda"),
        slots_p=dev(slots_p), bt_p=dev(bt_p), lens_p=dev(np.array([P_LEN], np.int32)),
        cu=dev(np.array([0, P_Q], np.int32)),
        q=torch.zeros((B, HQ, D), dtype=torch.bfloat16, device="cuda"),
        k_new=torch.zeros((B, HKV, D), device="cuda"),
        v_new=torch.zeros((B, HKV, D), device="cuda"),
        bt_d=dev(bt_d), lens_d=dev(np.asarray(BASE, np.int32) + 1),
        ks_d=dev(ks_d), vs_d=dev(vs_d),
        sm=float(np.float32(1.0 / math.sqrt(D))), max_len=max_len, splits_a=splits_a,
    )
    gen = torch.Generator(device="cuda").manual_seed(29)
    eager = Path(torch, fa, cache_d, cache_p, splits_a)
    graphed = Path(torch, fa, cache_d, cache_p, splits_a)
    _refresh(torch, x, gen)

    # warm-up of both copies on a side stream, then the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(fa, x, eager)
        _run(fa, x, graphed)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(fa, x, graphed)
    torch.cuda.synchronize()

    names = ["prefill out", "append+decode out", "many-split decode out", "k_scale", "v_scale",
             "decode cache", "prefill cache"]
    for step in range(STEPS):
        log(f"[graph] step {step} lens={(np.asarray(BASE) + step + 1).tolist()}")
        if step > 0:
            _refresh(torch, x, gen)
            x["lens_d"].add_(1)
        torch.cuda.synchronize()
        _run(fa, x, eager)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, eager.state(), graphed.state()):
            assert np.array_equal(_bits(a), _bits(b)), f"step {step}: {name} differs from eager"
        assert torch.isfinite(graphed.out_p).all() and torch.isfinite(graphed.out_d).all()
    graph.reset()
