"""CPU oracle for FP8-e4m3 paged-KV attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) imports, calls or links anything in this package; only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP path: the only inputs
both sides see come from the seeded generators in ``workloads``.

Everything is plain NumPy in float64 (float32 only where the method itself
fixes a float32 step, e.g. the quotient x / scale before encoding).

Pages cited (by title; section names as they appear on each page):

* [BLOG]  "State of FP8 KV-Cache and Attention Quantization in vLLM"
  (vLLM Blog, 2026-04-22; Chinese copy at shilu.ai).  The authority on
  the method.
* [SUMMARY] "vLLM FP8 KV-Cache と Attention 量子化のアップデート"
  (agentlenshq.com summary of the same post).
* [EXPLAINER] "KV Cache量子化とは？FP8でLLMの同時実行数を増やす前に測ること"
  (vasteelab.pages.dev, 2026-10-07).
* [GPUSTACK] "量子化が vLLM の推論性能に与える影響" (docs.gpustack.ai).

The pages name the e4m3 format but never define its bits; the codec follows
the OCP 8-bit floating point specification (OFP8), E4M3 variant, whose
largest finite value 448 matches the absmax/448 scales of the workloads.

Modules
-------
e4m3       encode / decode of OCP E4M3 codes (round-to-nearest-even,
           saturating), bf16 round-to-nearest-even.
quant      per-KV-head row quantization and the paged cache write.
attention  decode (split-KV + log-sum-exp combine is checked against the
           plain softmax definition) and the two prefill references.

Parity status of every function is stated in its docstring; all of them are
pinned by ``tests/test_oracle_*.py`` against values that do not come from the
oracle itself (hand-derived code values, an independent brute-force encoder,
torch's float8/bfloat16 casts, closed forms and literal loops).
"""

from . import e4m3, quant, attention  # noqa: F401
