"""Markdown tables of rocprofv3 kernel timings, for the profile notes.

Usage:
    python -m nvfp4_w4a4_quantized_amd.kernel_stats STATS_CSV [MAX_ROWS]
        the --stats summary (KERNEL_DISPATCH rows of *_kernel_stats.csv)
    python -m nvfp4_w4a4_quantized_amd.kernel_stats --last N TRACE_CSV [MAX_ROWS]
        from the --kernel-trace records (*_kernel_trace.csv): per kernel and
        grid size, the last N dispatches only (the steps a benchmark times,
        after its warm-up)
    python -m nvfp4_w4a4_quantized_amd.kernel_stats --window NAME GRID START COUNT TRACE_CSV
        the dispatches START .. START + COUNT - 1 (in time order) of the
        kernel whose name contains NAME, at grid size GRID
    python -m nvfp4_w4a4_quantized_amd.kernel_stats --span FIRST LAST N TRACE_CSV
        the time from the start of a dispatch of the kernel whose name
        contains FIRST to the end of the next dispatch whose name contains
        LAST (a stage of back-to-back launches): median, min and max over the
        last N such spans
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


def _dispatches(path: str):
    """{(short name, grid size): [(start, duration ns), ...]} of a trace."""
    groups = {}
    for r in csv.DictReader(open(path)):
        grid = int(r["Grid_Size"]) if "Grid_Size" in r else int(r["Grid_Size_X"])   # 1-D launches
        key = (_short(r["Kernel_Name"]), grid)
        groups.setdefault(key, []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return groups


def window(path: str, name: str, grid: int, start: int, count: int) -> str:
    for (kn, g), ds in _dispatches(path).items():
        if name in kn and g == grid:
            d = [v for _, v in sorted(ds)[start:start + count]]
            return "`%s` grid %d, dispatches %d-%d of %d: average %.1f us, min %.1f, max %.1f" % (
                kn, g, start, start + len(d) - 1, len(ds), sum(d) / len(d) / 1e3, min(d) / 1e3,
                max(d) / 1e3)
    raise SystemExit(f"no kernel containing {name!r} at grid {grid}")


def last_table(path: str, last: int, max_rows: int = 16) -> str:
    groups = _dispatches(path)
    rows = []
    for (name, grid), ds in groups.items():
        ds.sort()
        d = [v for _, v in ds[-last:]]
        rows.append((sum(d), name, grid, len(ds), d))
    rows.sort(key=lambda t: -t[0])
    out = ["| Kernel | Grid | Calls | Last | Average (us) | Min (us) | Max (us) |",
           "|---|---|---|---|---|---|---|"]
    for _, name, grid, n, d in rows[:max_rows]:
        out.append("| `%s` | %d | %d | %d | %.1f | %.1f | %.1f |" % (
            name, grid, n, len(d), sum(d) / len(d) / 1e3, min(d) / 1e3, max(d) / 1e3))
    return "\n".join(out)


def span(path: str, first: str, last: str, n: int) -> str:
    rows = []
    for r in csv.DictReader(open(path)):
        rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _short(r["Kernel_Name"])))
    rows.sort()
    spans, t0 = [], None
    for st, en, name in rows:
        if t0 is None and first in name:
            t0 = st
        if t0 is not None and last in name:
            spans.append(en - t0)
            t0 = None
    if not spans:
        raise SystemExit(f"no span from {first!r} to {last!r}")
    d = sorted(spans[-n:])
    return "%s .. %s, last %d of %d spans: median %.1f us, min %.1f, max %.1f" % (
        first, last, len(d), len(spans), d[len(d) // 2] / 1e3, d[0] / 1e3, d[-1] / 1e3)


if __name__ == "__main__":
    a = sys.argv[1:]
    if a and a[0] == "--last":
        print(last_table(a[2], int(a[1]), int(a[3]) if len(a) > 3 else 16))
    elif a and a[0] == "--span":
        print(span(a[4], a[1], a[2], int(a[3])))
    elif a and a[0] == "--window":
        print(window(a[5], a[1], int(a[2]), int(a[3]), int(a[4])))
    else:
        print(table(a[0], int(a[1]) if len(a) > 1 else 16))
