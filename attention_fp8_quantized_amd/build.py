"""Build libfa8attn.so in-tree with hipcc for gfx950.

Usage:  python -m attention_fp8_quantized_amd.build [--jobs N]

Each .hip translation unit is compiled to an object in parallel, then linked
into attention_fp8_quantized_amd/libfa8attn.so.  Flags:
  --offload-arch=gfx950     CDNA4 only, no other targets
  -O3 -std=c++17 -fPIC
  -fhip-fp32-correctly-rounded-divide-sqrt
                            x / scale in the cache write must be the correctly
                            rounded fp32 quotient (no fast-math anywhere)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                            no packed fp32 VALU instructions are generated
"""

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfa8attn.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "cache_write.hip", "decode.hip", "prefill.hip", "scales.hip",
           "stream_bench.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


def _compile(src):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    return src, r.returncode, msgs, obj


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    failed = False
    for src, rc, msgs, _ in results:
        if rc != 0 or (verbose and msgs):
            print(f"--- {src} (rc={rc})\n{msgs}", file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
           *[o for *_, o in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
