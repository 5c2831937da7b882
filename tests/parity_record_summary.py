"""Summarise a parity record (the JSON lines the GPU parity tests append to
$MOE_PARITY_RECORD: test name, per-tensor max|err|/max|ref|, per-tensor bar)
as a markdown table, plus the maximum error of each tensor over every test of
one comparison family (e.g. fp8_bwd/*/vs_quantised) beside its bar.

    MOE_PARITY_RECORD=gpurun_out/parity.jsonl python -m pytest tests -m gpu ...
    python tests/parity_record_summary.py gpurun_out/parity.jsonl
"""
from __future__ import annotations

import collections
import json
import sys


def family(test: str) -> str:
    """The test name without its shape parts (T..._H..., configN)."""
    parts = [p for p in test.split("/")
             if not ((p[:1] == "T" and p[1:2].isdigit()) or p.startswith("config"))]
    return "/".join(parts)


def main(path: str) -> None:
    rows = [json.loads(l) for l in open(path) if l.strip()]
    seen = {}
    for r in rows:                       # a test recorded twice keeps its last record
        seen[r["test"]] = r
    rows = list(seen.values())
    print(f"{len(rows)} recorded comparisons; error = max|gpu - ref| / max|ref| over the whole tensor.\n")
    print("## Maximum error per comparison family\n")
    print("| family | tensor | tests | max error | bar (at that max) | smallest bar/error |")
    print("|---|---|---|---|---|---|")
    fam = collections.defaultdict(list)
    for r in rows:
        for t, e in r["errors"].items():
            fam[(family(r["test"]), t)].append((e, r["bars"].get(t), r["test"]))
    for (f, t), v in sorted(fam.items()):
        emax, bar, _ = max(v, key=lambda x: x[0])
        ratios = [b / e for e, b, _ in v if b is not None and e > 0]
        rmin = f"{min(ratios):.1f}" if ratios else "-"
        print(f"| {f} | {t} | {len(v)} | {emax:.3g} | {bar if bar is None else f'{bar:.3g}'} | {rmin} |")
    print("\n## Every comparison\n")
    print("| test | tensor: error (bar) |")
    print("|---|---|")
    for r in sorted(rows, key=lambda r: r["test"]):
        cells = ", ".join(f"{t}: {e:.3g} ({r['bars'].get(t, float('nan')):.3g})" for t, e in r["errors"].items())
        print(f"| {r['test']} | {cells} |")


if __name__ == "__main__":
    main(sys.argv[1])
