"""Render the code/scale comparisons of a GPU test session as Markdown.

    KVQ_PARITY_REPORT=gpurun_out/parity_report.jsonl python -m pytest tests -m gpu
    python tests/parity_report.py gpurun_out/parity_report.jsonl > profiles/parity_mismatch_report.md

Each line of the input is one call of tests/parity.py compare_codes: the
test, the plan (rotation, D, G, code bits), the elements compared, and the
code and scale mismatches against the oracle's float32 decisions (the parity
bar) and against the plain definition with each exact quotient rounded once
(float64 decisions).
"""

from __future__ import annotations

import json
import sys


def render(path: str) -> str:
    recs = [json.loads(l) for l in open(path) if l.strip()]
    out = []
    n_el = sum(r["elements"] for r in recs)
    ident = [r for r in recs if r["rotation"] == "identity"]
    out.append(f"Comparisons: {len(recs)}, elements: {n_el:,}.")
    out.append("")
    out.append("| rotation | comparisons | elements | code mismatches | scale mismatches | fraction | "
               "code (fp64) | scale (fp64) | fraction (fp64) |")
    out.append("|---|---|---|---|---|---|---|---|---|")
    for rot in ("srft", "srht", "identity"):
        rs = [r for r in recs if r["rotation"] == rot]
        if not rs:
            continue
        e = sum(r["elements"] for r in rs)
        c, s = sum(r["code_mismatch"] for r in rs), sum(r["scale_mismatch"] for r in rs)
        c6, s6 = sum(r["code_mismatch_fp64"] for r in rs), sum(r["scale_mismatch_fp64"] for r in rs)
        out.append(f"| {rot} | {len(rs)} | {e:,} | {c} | {s} | {(c + s) / e:.2e} | {c6} | {s6} | "
                   f"{(c6 + s6) / e:.2e} |")
    out.append("")
    out.append(f"Unrotated (identity) comparisons: {len(ident)}, scale mismatches "
               f"{sum(r['scale_mismatch'] for r in ident)} (must be 0), code mismatches "
               f"{sum(r['code_mismatch'] for r in ident)} (each within the reciprocal band).")
    out.append("")
    out.append("Per comparison (fraction = (code + scale mismatches) / elements; the bar is < 1e-5 for int4 "
               "and < 1e-4 for int8 on samples of at least 10^6 elements):")
    out.append("")
    out.append("| test | rot | D | G | bits | elements | code | scale | fraction | code fp64 | scale fp64 | "
               "fraction fp64 |")
    out.append("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in recs:
        t = r["test"].replace("tests/", "").replace("|", "/")
        out.append(f"| {t} | {r['rotation']} | {r['D']} | {r['G']} | {r['bits']} | {r['elements']:,} | "
                   f"{r['code_mismatch']} | {r['scale_mismatch']} | {r['mismatch_frac']:.2e} | "
                   f"{r['code_mismatch_fp64']} | {r['scale_mismatch_fp64']} | {r['mismatch_frac_fp64']:.2e} |")
    return "\n".join(out)


if __name__ == "__main__":
    print(render(sys.argv[1]))
