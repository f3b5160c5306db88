"""C-ABI checks that need no GPU: the library loads, exports every function
that include/fa8attn.h declares, and rejects bad arguments on the host before
anything is launched."""

import ctypes
import os
import re

import pytest

import attention_fp8_quantized_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa8attn.h")

EINVAL, EUNSUPPORTED = 1, 2


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa8_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        pytest.fail("libfa8attn.so is not built (python -m attention_fp8_quantized_amd.build)")
    return fa.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"fa8_cache_write", "fa8_decode_attention", "fa8_prefill_attention"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in fa._SIGNATURES, f"binding lacks {n}"


def test_status_strings(lib):
    assert lib.fa8_status_string(0) == b"ok"
    assert lib.fa8_status_string(1) == b"invalid argument"
    assert lib.fa8_status_string(99) == b"unknown status"


def test_kv_tile_contract(lib):
    for d in (64, 128, 256):
        t = lib.fa8_prefill_kv_tile(d)
        assert t > 0 and t % 16 == 0
    assert lib.fa8_prefill_kv_tile(96) == 0


def _ws_expected(B, Hq, D, S):
    """Documented layout: int32 counters B*Hq*C, each on a 256-byte line,
    with C = 2 for S <= 64 and ceil(S/16) + 2 beyond; fp32 o_part
    B*Hq*S*D, m and l B*Hq*S (each array 16-byte aligned)."""
    a16 = lambda x: (x + 15) // 16 * 16  # noqa: E731
    c = 2 if S <= 64 else -(-S // 16) + 2
    return B * Hq * c * 256 + a16(B * Hq * S * D * 4) + 2 * a16(B * Hq * S * 4)


def test_workspace_size(lib):
    assert lib.fa8_decode_workspace_bytes(1, 32, 128, 64) == \
        32 * 2 * 256 + 32 * 64 * 128 * 4 + 2 * 32 * 64 * 4
    assert lib.fa8_decode_workspace_bytes(1, 1, 64, 1) == 2 * 256 + 256 + 16 + 16
    # 256 splits: 16 group counters + the set and merger counters
    assert lib.fa8_decode_workspace_bytes(1, 8, 256, 256) == \
        8 * 18 * 256 + 8 * 256 * 256 * 4 + 2 * 8 * 256 * 4
    for B, Hq, D, S in [(3, 5, 64, 65), (2, 7, 128, 100), (1, 1, 256, 250), (8, 64, 64, 2)]:
        assert lib.fa8_decode_workspace_bytes(B, Hq, D, S) == _ws_expected(B, Hq, D, S)
    assert lib.fa8_decode_workspace_bytes(0, 1, 64, 1) == 0


def test_num_splits_bounds(lib):
    assert lib.fa8_decode_num_splits(1, 8, 0, 0) == 1
    s = lib.fa8_decode_num_splits(1, 8, 32768, 0)
    assert 1 <= s <= 256
    # at least 8 pages (one per wave) per split
    assert lib.fa8_decode_num_splits(1, 8, 64, 0) == 1
    assert lib.fa8_decode_num_splits(1, 1, 16 * 16, 0) == 2
    assert lib.fa8_decode_num_splits(1, 1, 16 * 15, 0) == 1
    # a 128-token window never needs more than ceil(128/16)+1 pages
    assert lib.fa8_decode_num_splits(8, 8, 20000, 128) <= 2


def _p(x):
    return ctypes.c_void_p(x)


def _gpu_visible():
    # counting devices does not initialise the GPU runtime
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


# The argument-rejection tests below pass made-up device addresses with
# otherwise plausible shapes: only the host-side checks keep each call from
# launching.  Where a GPU is visible a regressed check would launch a kernel
# on those addresses, so they run only where no GPU is (the CPU suite).
fake_pointers = pytest.mark.skipif(_gpu_visible(),
                                   reason="made-up device pointers: CPU-only test")


@fake_pointers
def test_cache_write_rejects_bad_arguments(lib):
    fake = _p(0x1000)
    # bad input dtype
    assert lib.fa8_cache_write(fake, fake, 2, 1, 1, 64, fake, fake, fake, fake, 2, 1, None) == EINVAL
    assert b"in_dtype" in lib.fa8_last_error()
    # unsupported head_dim
    assert lib.fa8_cache_write(fake, fake, 0, 1, 1, 96, fake, fake, fake, fake, 2, 1, None) == EUNSUPPORTED
    # null pointers
    assert lib.fa8_cache_write(None, fake, 0, 1, 1, 64, fake, fake, fake, fake, 2, 1, None) == EINVAL
    # e4m3 cache without scales
    assert lib.fa8_cache_write(fake, fake, 0, 1, 1, 64, fake, None, None, fake, 2, 1, None) == EINVAL
    # n_tokens == 0 is a no-op (nothing launched)
    assert lib.fa8_cache_write(None, None, 0, 0, 1, 64, None, None, None, None, 2, 0, None) == 0
    assert lib.fa8_last_error() == b""



@fake_pointers
def test_last_error_is_per_thread(lib):
    # one thread's failure message is not visible to, nor overwritten by,
    # another thread's calls
    import threading
    fake = _p(0x1000)
    gate1, gate2 = threading.Barrier(2), threading.Barrier(2)
    seen = {}

    def fail_dtype():
        assert lib.fa8_cache_write(fake, fake, 2, 1, 1, 64, fake, fake, fake, fake, 2, 1, None) == EINVAL
        gate1.wait()          # the other thread fails now
        gate2.wait()
        seen["a"] = lib.fa8_last_error()

    def fail_head_dim():
        gate1.wait()
        assert lib.fa8_cache_write(fake, fake, 0, 1, 1, 96, fake, fake, fake, fake, 2, 1, None) == EUNSUPPORTED
        seen["b"] = lib.fa8_last_error()
        gate2.wait()

    def clean():
        seen["c"] = lib.fa8_last_error()

    ts = [threading.Thread(target=f) for f in (fail_dtype, fail_head_dim, clean)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(30)
    assert b"in_dtype" in seen["a"] and b"96" not in seen["a"]
    assert b"96" in seen["b"] and b"in_dtype" not in seen["b"]
    assert seen["c"] == b""

def _decode(lib, **over):
    fake = _p(0x1000)
    a = dict(q=fake, B=1, Hq=8, cache=fake, cd=2, nb=4, Hkv=2, D=64, bt=fake, mb=4,
             lens=fake, maxlen=64, ks=fake, vs=fake, sm=0.125, window=0, splits=1,
             out=fake, ws=_p(0x2000), wsb=1 << 20, stream=None)
    a.update(over)
    return lib.fa8_decode_attention(a["q"], a["B"], a["Hq"], a["cache"], a["cd"], a["nb"],
                                    a["Hkv"], a["D"], a["bt"], a["mb"], a["lens"], a["maxlen"],
                                    a["ks"], a["vs"], a["sm"], a["window"], a["splits"],
                                    a["out"], a["ws"], a["wsb"], a["stream"])


@fake_pointers
def test_decode_rejects_bad_arguments(lib):
    assert _decode(lib, Hq=7) == EINVAL                      # not a multiple of H_kv
    assert _decode(lib, Hq=6, Hkv=2) == EUNSUPPORTED         # G = 3
    assert _decode(lib, D=96) == EUNSUPPORTED
    assert _decode(lib, cd=0) == EINVAL
    assert _decode(lib, cd=4) == EINVAL
    assert _decode(lib, cd=3, ks=None) == EINVAL             # e5m2 needs scales too
    assert _decode(lib, maxlen=65) == EINVAL                 # 4 blocks hold 64 tokens
    assert _decode(lib, wsb=100) == EINVAL
    assert b"workspace" in lib.fa8_last_error()
    assert _decode(lib, ws=_p(0x2004)) == EINVAL             # misaligned
    assert _decode(lib, q=None) == EINVAL
    assert _decode(lib, ks=None) == EINVAL                   # e4m3 needs scales
    assert _decode(lib, sm=float("inf")) == EINVAL
    assert _decode(lib, splits=-1) == EINVAL
    assert _decode(lib, splits=257) == EINVAL
    assert _decode(lib, B=65536) == EUNSUPPORTED             # grid z extent
    assert _decode(lib, B=65535, wsb=100) == EINVAL          # ...65535 passes that check
    assert _decode(lib, B=0) == 0                            # empty batch: no-op


def _decode_noalloc(lib, **over):
    fake = _p(0x1000)
    a = dict(q=fake, B=1, Hq=8, cache=fake, cd=2, nb=4, Hkv=2, D=64, bt=fake, mb=4,
             lens=fake, maxlen=64, ks=fake, vs=fake, sm=0.125, window=0, splits=1,
             out=fake, stream=None)
    a.update(over)
    return lib.fa8_decode_attention_noalloc(a["q"], a["B"], a["Hq"], a["cache"], a["cd"],
                                            a["nb"], a["Hkv"], a["D"], a["bt"], a["mb"],
                                            a["lens"], a["maxlen"], a["ks"], a["vs"], a["sm"],
                                            a["window"], a["splits"], a["out"], a["stream"])


@fake_pointers
def test_decode_noalloc_rejects_bad_arguments_and_oversized_layouts(lib):
    # the same checks as the workspace entry point ...
    assert _decode_noalloc(lib, Hq=7) == EINVAL
    assert _decode_noalloc(lib, D=96) == EUNSUPPORTED
    assert _decode_noalloc(lib, q=None) == EINVAL
    assert _decode_noalloc(lib, splits=257) == EINVAL
    assert _decode_noalloc(lib, B=0) == 0                    # empty batch: no-op
    # ... and layouts beyond the fixed scratch: 64 x 16 heads x 256 splits
    # of 256 floats need 270 MB of partials (and 18,432 counters)
    assert _decode_noalloc(lib, B=64, Hq=16, Hkv=1, D=256, splits=256) == EINVAL
    assert b"scratch" in lib.fa8_last_error()
    # partials alone too large: 8 x 32 heads x 256 splits x 128 floats
    # (33.6 MB), counters small
    assert _decode_noalloc(lib, B=8, Hq=32, Hkv=8, D=128, splits=256) == EINVAL
    assert b"scratch" in lib.fa8_last_error()
    # counters alone too large: 4096 heads at one split (2 counters each)
    assert _decode_noalloc(lib, B=256, Hq=16, Hkv=16, D=64, splits=1) == EINVAL
    assert b"counter" in lib.fa8_last_error()


def _decode_append(lib, **over):
    fake = _p(0x1000)
    a = dict(q=fake, kn=fake, vn=fake, idt=0, B=1, Hq=8, cache=fake, cd=2, nb=4, Hkv=2, D=64,
             bt=fake, mb=4, lens=fake, maxlen=64, ks=fake, vs=fake, sm=0.125, window=0,
             splits=1, out=fake, ws=_p(0x2000), wsb=1 << 20, stream=None)
    a.update(over)
    return lib.fa8_decode_attention_append(
        a["q"], a["kn"], a["vn"], a["idt"], a["B"], a["Hq"], a["cache"], a["cd"], a["nb"],
        a["Hkv"], a["D"], a["bt"], a["mb"], a["lens"], a["maxlen"], a["ks"], a["vs"], a["sm"],
        a["window"], a["splits"], a["out"], a["ws"], a["wsb"], a["stream"])


@fake_pointers
def test_decode_append_rejects_bad_arguments(lib):
    assert _decode_append(lib, idt=2) == EINVAL              # e4m3 is not an input type
    assert _decode_append(lib, kn=None) == EINVAL
    assert _decode_append(lib, vn=None) == EINVAL
    assert _decode_append(lib, D=96) == EUNSUPPORTED         # decode checks still apply
    assert _decode_append(lib, wsb=100) == EINVAL
    assert _decode_append(lib, B=0, kn=None, vn=None) == 0   # empty batch: no-op


@fake_pointers
def test_prefill_rejects_bad_arguments(lib):
    fake = _p(0x1000)

    def call(**over):
        a = dict(q=fake, cu=fake, B=1, Hq=8, mq=16, cache=fake, cd=2, nb=4, Hkv=2, D=64,
                 bt=fake, mb=4, lens=fake, qs=fake, ks=fake, vs=fake, sm=0.125, window=0,
                 acc=1, out=fake)
        a.update(over)
        return lib.fa8_prefill_attention(a["q"], a["cu"], a["B"], a["Hq"], a["mq"], a["cache"],
                                         a["cd"], a["nb"], a["Hkv"], a["D"], a["bt"], a["mb"],
                                         a["lens"],
                                         a["qs"], a["ks"], a["vs"], a["sm"], a["window"],
                                         a["acc"], a["out"], None)

    assert call(Hq=7) == EINVAL
    assert call(D=80) == EUNSUPPORTED
    assert call(acc=-1) == EINVAL
    assert call(acc=65537) == EINVAL
    assert call(cd=1) == EINVAL                  # prefill needs an FP8 cache
    assert call(cd=4) == EINVAL
    assert call(qs=None) == EINVAL
    assert call(B=65536) == EUNSUPPORTED         # grid z extent
    assert call(Hq=65536 * 2, Hkv=2) == EUNSUPPORTED   # grid y extent
    assert call(B=0) == 0


@fake_pointers
def test_absmax_scales_rejects_bad_arguments(lib):
    fake = _p(0x1000)

    def call(**over):
        a = dict(k=fake, v=fake, idt=0, n=4, H=2, D=64, cd=2, ks=fake, vs=fake)
        a.update(over)
        return lib.fa8_absmax_scales(a["k"], a["v"], a["idt"], a["n"], a["H"], a["D"], a["cd"],
                                     a["ks"], a["vs"], None)

    assert call(idt=2) == EINVAL                 # e4m3 is not an input type
    assert call(cd=1) == EINVAL                  # a bf16 cache takes no scales
    assert call(cd=4) == EINVAL
    assert call(H=0) == EINVAL
    assert call(H=4097) == EINVAL
    assert call(D=96) == EUNSUPPORTED
    assert call(ks=None) == EINVAL
    assert call(k=None) == EINVAL
    assert call(n=-1) == EINVAL


def test_missing_library_raises_and_nothing_falls_back(monkeypatch, tmp_path):
    # with no library every call raises: there is no host implementation
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "library_path", lambda: str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        fa.load()
    with pytest.raises(RuntimeError):
        fa.decode_num_splits(1, 8, 1024)
    with pytest.raises(RuntimeError):
        fa.prefill_kv_tile(128)


def test_host_tensors_are_rejected(lib):
    # the binding passes device pointers only; host tensors are refused before
    # any call into the library
    torch = pytest.importorskip("torch")
    cache = torch.zeros((4, 2, 2, 16, 64), dtype=torch.uint8)
    q = torch.zeros((1, 8, 64), dtype=torch.bfloat16)
    bt = torch.zeros((1, 4), dtype=torch.int32)
    lens = torch.ones(1, dtype=torch.int32)
    sc = torch.ones(2, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.decode_attention(q, cache, bt, lens, sc, sc, 0.125, 16, num_splits=1)
    k = torch.zeros((3, 2, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.cache_write(k, k, torch.zeros(3, dtype=torch.int64), sc, sc, cache)
