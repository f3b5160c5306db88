"""Python binding of libfa8attn.so (FP8 paged-KV attention for gfx950: e4m3 or
e5m2 cache codes with per-KV-head scales, or a bf16 cache).

Argument marshalling only: every step runs in the library's HIP kernels.
torch supplies device memory (``data_ptr``) and the stream
(``torch.cuda.current_stream()``); nothing here computes on tensor values.
If the library is missing the import of this module still works, but every
call raises ``RuntimeError`` (there is no fallback path).

Names follow the C ABI in include/fa8attn.h:
    cache_write, absmax_scales, decode_num_splits, decode_workspace_bytes,
    decode_attention, decode_attention_noalloc, decode_attention_append, prefill_kv_tile,
    prefill_attention, stream_read, stream_copy
"""

import ctypes
import os

__all__ = [
    "FA8_F32", "FA8_BF16", "FA8_E4M3", "FA8_E5M2", "BLOCK_SIZE", "Fa8Error", "library_path",
    "load", "cache_write", "absmax_scales", "decode_num_splits", "decode_workspace_bytes",
    "decode_attention", "decode_attention_noalloc", "decode_attention_append",
    "prefill_kv_tile", "prefill_attention", "new_cache",
    "new_decode_workspace",
]

FA8_F32, FA8_BF16, FA8_E4M3, FA8_E5M2 = 0, 1, 2, 3
_FP8 = (FA8_E4M3, FA8_E5M2)
BLOCK_SIZE = 16
_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.path.join(_HERE, "libfa8attn.so")


class Fa8Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"fa8attn status {status}: {message}")
        self.status = status


_lib = None
_VP, _I32, _I64, _F32, _SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                              ctypes.c_float, ctypes.c_size_t)

_SIGNATURES = {
    "fa8_cache_write": (_I32, [_VP, _VP, _I32, _I64, _I32, _I32, _VP, _VP, _VP, _VP,
                               _I32, _I64, _VP]),
    "fa8_absmax_scales": (_I32, [_VP, _VP, _I32, _I64, _I32, _I32, _I32, _VP, _VP, _VP]),
    "fa8_decode_num_splits": (_I32, [_I32, _I32, _I32, _I32]),
    "fa8_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "fa8_decode_attention": (_I32, [_VP, _I32, _I32, _VP, _I32, _I64, _I32, _I32, _VP,
                                    _I32, _VP, _I32, _VP, _VP, _F32, _I32, _I32, _VP,
                                    _VP, _SZ, _VP]),
    "fa8_decode_attention_noalloc": (_I32, [_VP, _I32, _I32, _VP, _I32, _I64, _I32, _I32, _VP,
                                            _I32, _VP, _I32, _VP, _VP, _F32, _I32, _I32, _VP,
                                            _VP]),
    "fa8_decode_attention_append": (_I32, [_VP, _VP, _VP, _I32, _I32, _I32, _VP, _I32, _I64,
                                            _I32, _I32, _VP, _I32, _VP, _I32, _VP, _VP, _F32,
                                            _I32, _I32, _VP, _VP, _SZ, _VP]),
    "fa8_prefill_kv_tile": (_I32, [_I32]),
    "fa8_prefill_attention": (_I32, [_VP, _VP, _I32, _I32, _I32, _VP, _I32, _I64, _I32, _I32,
                                     _VP, _I32, _VP, _VP, _VP, _VP, _F32, _I32, _I32,
                                     _VP, _VP]),
    "fa8_stream_read": (_I32, [_VP, _SZ, _VP, _VP]),
    "fa8_stream_copy": (_I32, [_VP, _VP, _SZ, _VP]),
    "fa8_status_string": (ctypes.c_char_p, [_I32]),
    "fa8_last_error": (ctypes.c_char_p, []),
}


def load():
    """Load libfa8attn.so once and return the ctypes handle (raises if absent)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built: run `python -m attention_fp8_quantized_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status):
    if status != 0:
        lib = load()
        raise Fa8Error(status, lib.fa8_last_error().decode())


_torch_mod = None


def _torch():
    global _torch_mod
    if _torch_mod is None:
        import torch
        _torch_mod = torch
    return _torch_mod


def _ptr(t):
    # ctypes takes a plain int for a c_void_p argument
    return None if t is None else t.data_ptr()


def _stream(t):
    """The current stream of t's device as an integer handle.  torch's raw
    accessor skips building a Stream object (about 2 us per call); the
    public call is the fallback."""
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(t.device.index if t.device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _require(t, name, dtype=None, device=None, ndim=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")


def _cache_dtype(cache):
    """fa8_dtype of a cache tensor: uint8 or float8_e4m3fn holds e4m3 codes,
    float8_e5m2 e5m2 codes, bfloat16 (or 16-bit integers) bf16 values."""
    torch = _torch()
    if cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FA8_E4M3
    if cache.dtype == torch.float8_e5m2:
        return FA8_E5M2
    if cache.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return FA8_BF16
    raise ValueError("cache must be uint8 / float8_e4m3fn (e4m3 codes), float8_e5m2 "
                     "(e5m2 codes) or bfloat16")


def new_cache(num_blocks, num_kv_heads, head_dim, cache_dtype="e4m3", device="cuda"):
    """Allocate a paged cache tensor [num_blocks][H_kv][2][16][head_dim]:
    uint8 codes for 'e4m3', float8_e5m2 codes for 'e5m2', bfloat16 for
    'bf16'."""
    torch = _torch()
    dts = {"e4m3": torch.uint8, "e5m2": torch.float8_e5m2, "bf16": torch.bfloat16}
    if cache_dtype not in dts:
        raise ValueError(f"cache_dtype must be one of {sorted(dts)}")
    dt = dts[cache_dtype]
    return torch.empty((num_blocks, num_kv_heads, 2, BLOCK_SIZE, head_dim),
                       dtype=dt, device=device)


def cache_write(k, v, slot_mapping, k_scale, v_scale, cache):
    """Quantise (FP8 cache) or round (bf16 cache) k/v [N][H_kv][D] into the
    paged cache at ``slot_mapping`` (int64 [N]; negative = skip)."""
    torch = _torch()
    _require(cache, "cache", ndim=5)
    dev = cache.device
    nb, hkv, two, bs, d = cache.shape
    if two != 2 or bs != BLOCK_SIZE:
        raise ValueError("cache must be [num_blocks][H_kv][2][16][D]")
    _require(k, "k", device=dev, ndim=3)
    _require(v, "v", dtype=k.dtype, device=dev, ndim=3)
    if k.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("k/v must be float32 or bfloat16")
    if tuple(k.shape[1:]) != (hkv, d) or k.shape != v.shape:
        raise ValueError(f"k/v must be [N][{hkv}][{d}]")
    _require(slot_mapping, "slot_mapping", dtype=torch.int64, device=dev, ndim=1)
    if slot_mapping.shape[0] != k.shape[0]:
        raise ValueError("slot_mapping must have one entry per row")
    cdt = _cache_dtype(cache)
    if cdt in _FP8:
        for s, nm in ((k_scale, "k_scale"), (v_scale, "v_scale")):
            _require(s, nm, dtype=torch.float32, device=dev, ndim=1)
            if s.shape[0] != hkv:
                raise ValueError(f"{nm} must have {hkv} entries")
    lib = load()
    _check(lib.fa8_cache_write(
        _ptr(k), _ptr(v), FA8_BF16 if k.dtype == torch.bfloat16 else FA8_F32,
        k.shape[0], hkv, d, _ptr(slot_mapping),
        _ptr(k_scale) if cdt in _FP8 else None,
        _ptr(v_scale) if cdt in _FP8 else None,
        _ptr(cache), cdt, nb, _stream(cache)))


def absmax_scales(k, v, k_scale=None, v_scale=None, cache_dtype="e4m3"):
    """Per-KV-head scales of k/v [N][H_kv][D] (float32 or bfloat16) for an FP8
    cache: max(fl32(absmax_h / F), 2^-126) over the finite entries of head
    h, F = 448 ('e4m3') or 57344 ('e5m2'), computed on the device.  Writes into ``k_scale``/``v_scale`` (float32
    [H_kv]) when given, else allocates them; returns (k_scale, v_scale)."""
    torch = _torch()
    _require(k, "k", ndim=3)
    dev = k.device
    _require(v, "v", dtype=k.dtype, device=dev, ndim=3)
    if k.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("k/v must be float32 or bfloat16")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    n, hkv, d = k.shape
    fmts = {"e4m3": FA8_E4M3, "e5m2": FA8_E5M2}
    if cache_dtype not in fmts:
        raise ValueError(f"no scales for cache_dtype {cache_dtype!r}")
    out = []
    for s, nm in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if s is None:
            s = torch.empty(hkv, dtype=torch.float32, device=dev)
        _require(s, nm, dtype=torch.float32, device=dev, ndim=1)
        if s.shape[0] != hkv:
            raise ValueError(f"{nm} must have {hkv} entries")
        out.append(s)
    _check(load().fa8_absmax_scales(
        _ptr(k), _ptr(v), FA8_BF16 if k.dtype == torch.bfloat16 else FA8_F32, n, hkv, d,
        fmts[cache_dtype], _ptr(out[0]), _ptr(out[1]), _stream(k)))
    return out[0], out[1]


def decode_num_splits(batch, num_kv_heads, max_seq_len, window=0):
    return int(load().fa8_decode_num_splits(batch, num_kv_heads, max_seq_len, window))


_ws_bytes = {}


def decode_workspace_bytes(batch, num_q_heads, head_dim, num_splits):
    key = (batch, num_q_heads, head_dim, num_splits)
    n = _ws_bytes.get(key)
    if n is None:
        n = int(load().fa8_decode_workspace_bytes(batch, num_q_heads, head_dim, num_splits))
        if len(_ws_bytes) < 4096:
            _ws_bytes[key] = n
    return n


def new_decode_workspace(nbytes, device="cuda"):
    """Zero-filled decode workspace of ``nbytes`` (the library needs it zeroed
    once; every decode call leaves it reusable)."""
    torch = _torch()
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device)


_NO_WORKSPACE = object()   # the allocation-free entry point takes none


def _decode_args(q, cache, block_table, seq_lens, k_scale, v_scale, max_seq_len, window,
                 num_splits, out, workspace):
    torch = _torch()
    _require(cache, "cache", ndim=5)
    dev = cache.device
    nb, hkv, _, _, d = cache.shape
    _require(q, "q", dtype=torch.bfloat16, device=dev, ndim=3)
    B, hq, dq = q.shape
    if dq != d:
        raise ValueError("q head_dim does not match the cache")
    _require(block_table, "block_table", dtype=torch.int32, device=dev, ndim=2)
    _require(seq_lens, "seq_lens", dtype=torch.int32, device=dev, ndim=1)
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table / seq_lens must have one row per sequence")
    cdt = _cache_dtype(cache)
    if cdt in _FP8:
        _require(k_scale, "k_scale", dtype=torch.float32, device=dev, ndim=1)
        _require(v_scale, "v_scale", dtype=torch.float32, device=dev, ndim=1)
    splits = num_splits or decode_num_splits(B, hkv, int(max_seq_len), int(window))
    if workspace is _NO_WORKSPACE:
        workspace = None
    elif workspace is None:
        workspace = new_decode_workspace(decode_workspace_bytes(B, hq, d, splits), dev)
    else:
        _require(workspace, "workspace", device=dev)
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.float32, device=dev)
    else:
        _require(out, "out", dtype=torch.float32, device=dev, ndim=3)
    head = (_ptr(q),)
    tail = (B, hq, _ptr(cache), cdt, nb, hkv, d, _ptr(block_table), block_table.shape[1],
            _ptr(seq_lens), int(max_seq_len),
            _ptr(k_scale) if cdt in _FP8 else None,
            _ptr(v_scale) if cdt in _FP8 else None)
    return head, tail, splits, out, workspace


def decode_attention(q, cache, block_table, seq_lens, k_scale, v_scale, sm_scale,
                     max_seq_len, window=0, num_splits=0, out=None, workspace=None):
    """One decode step. q bf16 [B][H_q][D] -> out fp32 [B][H_q][D].

    ``max_seq_len`` is a host-side upper bound of ``seq_lens`` (sizes the
    grid).  ``workspace`` (uint8 device tensor from ``new_decode_workspace``)
    is allocated here when not given; pass one to keep the call
    allocation-free."""
    lib = load()
    head, tail, splits, out, workspace = _decode_args(
        q, cache, block_table, seq_lens, k_scale, v_scale, max_seq_len, window, num_splits,
        out, workspace)
    _check(lib.fa8_decode_attention(
        *head, *tail, float(sm_scale), int(window), int(splits), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(cache)))
    return out


def decode_attention_noalloc(q, cache, block_table, seq_lens, k_scale, v_scale, sm_scale,
                             max_seq_len, out, window=0, num_splits=0):
    """decode_attention without a workspace: the library's fixed per-GPU
    scratch holds the split partials, so the call allocates nothing (``out``
    is required).  Calls that overlap on one GPU share that scratch and must
    be ordered on one stream."""
    lib = load()
    _require(out, "out")
    head, tail, splits, out, _ = _decode_args(
        q, cache, block_table, seq_lens, k_scale, v_scale, max_seq_len, window, num_splits,
        out, _NO_WORKSPACE)
    _check(lib.fa8_decode_attention_noalloc(
        *head, *tail, float(sm_scale), int(window), int(splits), _ptr(out), _stream(cache)))
    return out


def decode_attention_append(q, k_new, v_new, cache, block_table, seq_lens, k_scale, v_scale,
                            sm_scale, max_seq_len, window=0, num_splits=0, out=None,
                            workspace=None):
    """Fused decode step: writes k_new / v_new ([B][H_kv][D], fp32 or bf16)
    as token seq_lens[b]-1 of each sequence (the bytes cache_write would
    store) and attends over the context including it."""
    torch = _torch()
    lib = load()
    head, tail, splits, out, workspace = _decode_args(
        q, cache, block_table, seq_lens, k_scale, v_scale, max_seq_len, window, num_splits,
        out, workspace)
    B, hkv, d = q.shape[0], cache.shape[1], cache.shape[4]
    if k_new.dtype not in (torch.float32, torch.bfloat16) or v_new.dtype != k_new.dtype:
        raise ValueError("k_new / v_new must both be float32 or both bfloat16")
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        _require(t, name, device=cache.device, ndim=3)
        if tuple(t.shape) != (B, hkv, d):
            raise ValueError(f"{name} must be [batch, num_kv_heads, head_dim]")
    in_dtype = FA8_BF16 if k_new.dtype == torch.bfloat16 else FA8_F32
    _check(lib.fa8_decode_attention_append(
        head[0], _ptr(k_new), _ptr(v_new), in_dtype, *tail, float(sm_scale), int(window),
        int(splits), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(cache)))
    return out


def prefill_kv_tile(head_dim):
    return int(load().fa8_prefill_kv_tile(head_dim))


def prefill_attention(q, cu_q_lens, cache, block_table, seq_lens, q_scale, k_scale,
                      v_scale, sm_scale, max_q_len, window=0, accum_mode=1, out=None):
    """Causal FP8 prefill. q bf16 [T][H_q][D] (packed by ``cu_q_lens``) ->
    out fp32 [T][H_q][D].  ``seq_lens`` count the context including the
    chunk; ``q_scale`` is a 1-element fp32 device tensor."""
    torch = _torch()
    _require(cache, "cache", ndim=5)
    cdt = _cache_dtype(cache)
    if cdt not in _FP8:
        raise ValueError("prefill needs an FP8 (e4m3 or e5m2) cache")
    dev = cache.device
    nb, hkv, _, _, d = cache.shape
    _require(q, "q", dtype=torch.bfloat16, device=dev, ndim=3)
    T, hq, dq = q.shape
    if dq != d:
        raise ValueError("q head_dim does not match the cache")
    _require(cu_q_lens, "cu_q_lens", dtype=torch.int32, device=dev, ndim=1)
    B = cu_q_lens.shape[0] - 1
    _require(block_table, "block_table", dtype=torch.int32, device=dev, ndim=2)
    _require(seq_lens, "seq_lens", dtype=torch.int32, device=dev, ndim=1)
    for s, nm in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _require(s, nm, dtype=torch.float32, device=dev, ndim=1)
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.float32, device=dev)
    else:
        _require(out, "out", dtype=torch.float32, device=dev, ndim=3)
    lib = load()
    _check(lib.fa8_prefill_attention(
        _ptr(q), _ptr(cu_q_lens), B, hq, int(max_q_len), _ptr(cache), cdt, nb, hkv, d,
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), _ptr(q_scale),
        _ptr(k_scale), _ptr(v_scale), float(sm_scale), int(window), int(accum_mode),
        _ptr(out), _stream(cache)))
    return out


def stream_read(src, sink):
    """Read all of ``src`` (a contiguous CUDA tensor, nbytes % 16 == 0) once;
    ``sink`` is a CUDA tensor of >= 4 bytes."""
    _require(src, "src")
    _require(sink, "sink", device=src.device)
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold >= 4 bytes")
    lib = load()
    _check(lib.fa8_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                               _stream(src)))


def stream_copy(dst, src):
    """dst <- src bytewise (contiguous CUDA tensors of equal byte size)."""
    _require(src, "src")
    _require(dst, "dst", device=src.device)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("dst and src must have the same byte size")
    lib = load()
    _check(lib.fa8_stream_copy(_ptr(dst), _ptr(src), n, _stream(src)))
