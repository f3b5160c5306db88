"""Markdown table of the parity records the GPU tests write.

    FA8_PARITY_LOG=/tmp/parity.jsonl python -m pytest tests -m gpu
    python tests/parity_summary.py /tmp/parity.jsonl

Prints, for every gated comparison that carries a context length (decode
at 1k..128k, prefill chunks up to the last 32k chunk of a 128k fill, both
accumulation modes), the shape, context, mode and the measured errors
against the oracle.  Reads only the records; computes nothing new.
"""

import json
import sys


def rows(path):
    out = []
    with open(path) as f:
        for line in f:
            r = json.loads(line)
            if "kernel" in r and "context" in r:
                out.append(r)
    return out


def table(recs):
    lines = ["| kernel | shape | cache | context | chunk | accum_mode | compared | max_abs | "
             "rel_l2 | rel_l2 beyond flip allowance | worst row rel_l2 | gate |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    key = lambda r: (r["kernel"], r["shape"], r.get("cache", ""), r["context"],  # noqa: E731
                     r.get("chunk", 0), -1 if r.get("accum_mode") is None else
                     (r["accum_mode"] if r["accum_mode"] != 1 else -0.5))
    seen = set()
    for r in sorted(recs, key=key):
        k = (r["what"], r.get("accum_mode"))
        if k in seen:
            continue
        seen.add(k)
        lines.append(
            f"| {r['kernel']} | {r['shape']} | {r.get('cache', '')} | {r['context']} | "
            f"{r.get('chunk', '')} | {r.get('accum_mode', '')} | {r.get('compared', '')} | "
            f"{r['max_abs']:.2e} | {r['rel_l2']:.2e} | {r.get('rel_l2_excess', float('nan')):.2e} | "
            f"{r['worst_row_rel_l2']:.2e} | {'pass' if r['passed'] else 'FAIL'} |")
    return "\n".join(lines)


if __name__ == "__main__":
    print(table(rows(sys.argv[1] if len(sys.argv) > 1 else "parity.jsonl")))
