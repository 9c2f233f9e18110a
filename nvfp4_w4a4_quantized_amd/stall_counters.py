"""Issue and stall breakdown of the GEMM kernels from rocprofv3 counter passes.

Usage (run from the repository root, after passes such as
    rocprofv3 --pmc SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY \\
        SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES \\
        --output-format csv -d DIR1 -o p1 -- python3 bench.py ...
and two more with the other counters named below):
    python -m nvfp4_w4a4_quantized_amd.stall_counters CSV [CSV ...]

Dispatches are grouped by kernel name and grid size; the first of each group
is dropped as a warm-up and the others averaged, each counter over the passes
that collected it.  Per group it prints:
  - the shader clock: SQ_BUSY_CYCLES (summed over the shader engines) over
    the number of engines and the dispatch time;
  - MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs and the busy cycles;
  - the wave-time split of SQ_WAVE_CYCLES into SQ_WAIT_ANY (s_waitcnt and
    other waits), SQ_WAIT_INST_ANY (an instruction waiting to issue) and
    SQ_ACTIVE_INST_ANY (issuing);
  - VALU and LDS instructions per MFMA instruction (SQ_INSTS_VALU,
    SQ_INSTS_LDS, SQ_INSTS_MFMA);
  - the share of VALU issue cycles spent while the matrix core was busy:
    SQ_VALU_MFMA_COEXEC_CYCLES over four cycles per SQ_INSTS_VALU;
  - LDS activity per compute unit (SQ_LDS_IDX_ACTIVE) and its bank-conflict
    share (SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE).
"""
from __future__ import annotations

import csv
import re
import sys

SHADER_ENGINES = 32      # MI355X: 8 XCDs of 4 shader engines
SIMDS = 1024             # 256 compute units of 4 SIMDs
CUS = 256


def _short(name: str) -> str:
    name = name.split("(")[0].replace("void ", "").replace("nvfp4::", "")
    return re.sub(r"\s+", " ", name).strip()


def collect(paths):
    """{(kernel, grid size): [{counter: value, 'ns': duration}, ...]} per pass
    file, dispatches in order, GEMM kernels only."""
    groups = {}
    for path in paths:
        disp = {}
        for r in csv.DictReader(open(path)):
            if "gemm" not in r["Kernel_Name"]:
                continue
            key = (r["Kernel_Name"], int(r["Grid_Size"]), int(r["Dispatch_Id"]))
            d = disp.setdefault(key, {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        per = {}
        for key in sorted(disp, key=lambda k: k[2]):
            per.setdefault(key[:2], []).append(disp[key])
        for k, ds in per.items():
            groups.setdefault(k, []).append(ds[1:] if len(ds) > 1 else ds)
    return groups


def _mean(passes, counter):
    vals = [d[counter] for ds in passes for d in ds if counter in d]
    return sum(vals) / len(vals) if vals else float("nan")


def _mean_over(passes, counter, denom):
    """Mean over dispatches of counter / denom(dispatch) for the passes that
    hold the counter (each pass has its own dispatch times)."""
    vals = [d[counter] / denom(d) for ds in passes for d in ds if counter in d]
    return sum(vals) / len(vals) if vals else float("nan")


def table(paths) -> str:
    rows = ["| Kernel | Grid | Time (us) | Clock (GHz) | MFMA busy | Wait | Wait to issue | Issuing | "
            "VALU / MFMA | LDS / MFMA | VALU beside MFMA | LDS active / CU | LDS bank conflicts |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for (name, grid), passes in collect(paths).items():
        ns = sum(d["ns"] for ds in passes for d in ds) / sum(len(ds) for ds in passes)
        clock = _mean_over(passes, "SQ_BUSY_CYCLES", lambda d: SHADER_ENGINES * d["ns"])
        cycles = _mean(passes, "SQ_BUSY_CYCLES") / SHADER_ENGINES
        mfma_busy = _mean(passes, "SQ_VALU_MFMA_BUSY_CYCLES") / SIMDS / cycles
        wave = _mean(passes, "SQ_WAVE_CYCLES")
        valu, mfma, lds = (_mean(passes, c) for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS"))
        coexec = _mean(passes, "SQ_VALU_MFMA_COEXEC_CYCLES") / (4 * valu)
        idx = _mean(passes, "SQ_LDS_IDX_ACTIVE")
        # LDS activity is taken against the clock of the pass that held it
        lds_active = idx / CUS / (clock * ns) if clock == clock else float("nan")
        rows.append("| `%s` | %d | %.1f | %.2f | %.0f%% | %.0f%% | %.0f%% | %.0f%% | %.1f | %.2f | %.0f%% | %.0f%% | %.0f%% |" % (
            _short(name), grid, ns / 1e3, clock, 100 * mfma_busy,
            100 * _mean(passes, "SQ_WAIT_ANY") / wave, 100 * _mean(passes, "SQ_WAIT_INST_ANY") / wave,
            100 * _mean(passes, "SQ_ACTIVE_INST_ANY") / wave, valu / mfma, lds / mfma, 100 * coexec,
            100 * lds_active, 100 * _mean(passes, "SQ_LDS_BANK_CONFLICT") / idx))
    return "\n".join(rows)


def main(argv):
    if len(argv) < 2:
        print(__doc__)
        return 2
    print(table(argv[1:]))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
