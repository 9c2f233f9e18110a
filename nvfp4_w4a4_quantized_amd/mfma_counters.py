"""Matrix-core utilisation of the GEMM kernels from one rocprofv3 counter pass.

Usage (run from the repository root, after a pass such as
    rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_F16 --output-format csv -d DIR -o m -- python3 bench.py ...):
    python -m nvfp4_w4a4_quantized_amd.mfma_counters COUNTER_CSV [GFLOP_PER_KERNEL ...]

Per GEMM launch shape (dispatches grouped by kernel name and grid size, the
first one of each dropped as a warm-up) it prints:
  - MfmaUtil: the cycles the matrix ALU of a SIMD was busy, summed over all
    1024 SIMDs, over the dispatch's busy cycles times 1024, in percent;
  - the f16 MFMA work the hardware executed (SQ_INSTS_VALU_MFMA_MOPS_F16 counts
    it in units of 512 flops), against the algorithmic flops given as
    NAME=GFLOP arguments (NAME a substring of "kernel/grid size"), which exclude
    padding rows and the MFMAs of partly valid row blocks;
  - that executed work over the dispatch time of the counter run.
"""
from __future__ import annotations

import csv
import re
import sys


def _short(name: str) -> str:
    name = name.split("(")[0].replace("void ", "").replace("nvfp4::", "")
    return re.sub(r"\s+", " ", name).strip()


def per_dispatch(path: str):
    """{(kernel, grid size): [{counter: value, 'ns': duration}, ...]} in
    dispatch order."""
    disp = {}
    for r in csv.DictReader(open(path)):
        if "gemm" not in r["Kernel_Name"] and "single_pass" not in r["Kernel_Name"]:
            continue
        key = (r["Kernel_Name"], int(r["Grid_Size"]), int(r["Dispatch_Id"]))
        d = disp.setdefault(key, {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = {}
    for key in sorted(disp, key=lambda k: k[2]):
        out.setdefault(key[:2], []).append(disp[key])
    return out


def table(path: str, algorithmic: dict) -> str:
    rows = ["| Kernel | Grid | Dispatches | Time (us) | MfmaUtil | Executed f16 MFMA (GFLOP) | "
            "Algorithmic (GFLOP) | Executed rate (TFLOP/s) |",
            "|---|---|---|---|---|---|---|---|"]
    for (name, grid), ds in per_dispatch(path).items():
        ds = ds[1:] if len(ds) > 1 else ds
        n = len(ds)
        ns = sum(d["ns"] for d in ds) / n
        util = sum(d.get("MfmaUtil", float("nan")) for d in ds) / n
        gflop = sum(d.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) for d in ds) / n * 512 / 1e9
        alg = next((v for k, v in algorithmic.items() if k in "%s/%d" % (_short(name), grid)),
                   None)
        rows.append("| `%s` | %d | %d | %.1f | %.1f%% | %.1f | %s | %.0f |" % (
            _short(name), grid, n, ns / 1e3, util, gflop, "%.1f" % alg if alg else "-",
            gflop * 1e9 / (ns * 1e-9) / 1e12))
    return "\n".join(rows)


if __name__ == "__main__":
    alg = {}
    for a in sys.argv[2:]:
        k, v = a.rsplit("=", 1)
        alg[k] = float(v)
    print(table(sys.argv[1], alg))
