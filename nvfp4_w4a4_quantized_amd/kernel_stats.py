"""Markdown table of a rocprofv3 --stats kernel summary (KERNEL_DISPATCH
rows of the *_kernel_stats.csv file), for the profile notes.

Usage:
    python -m nvfp4_w4a4_quantized_amd.kernel_stats STATS_CSV [MAX_ROWS]
"""
from __future__ import annotations

import csv
import re
import sys


def _short(name: str) -> str:
    name = name.split("(")[0].replace("void ", "").replace("nvfp4::", "")
    return re.sub(r"\s+", " ", name).strip()


def table(path: str, max_rows: int = 16) -> str:
    rows = [r for r in csv.DictReader(open(path)) if r.get("Domain", "KERNEL_DISPATCH") ==
            "KERNEL_DISPATCH"]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share |",
           "|---|---|---|---|---|---|"]
    for r in rows[:max_rows]:
        out.append("| `%s` | %s | %.1f | %.1f | %.1f | %.1f%% |" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out)


if __name__ == "__main__":
    print(table(sys.argv[1], int(sys.argv[2]) if len(sys.argv) > 2 else 16))
