"""HBM traffic of the FC1 kernel from two rocprofv3 counter passes.

Usage (after the two passes described in profiles/; run from the repository
root):
    python -m nvfp4_w4a4_quantized_amd.traffic FETCH_CSV WRITE_CSV COPY_MIB OUT_JSON
    python -m nvfp4_w4a4_quantized_amd.traffic --kernels NAME FETCH_CSV WRITE_CSV COPY_MIB
        a table of the scaled fetch and write bytes per dispatch (mean over
        the dispatches after each kernel's first) of every kernel whose name
        contains NAME, per grid size

FETCH_SIZE and WRITE_SIZE are read per dispatch (KiB).  Each is scaled by the
ratio of the known bytes of the plain device copy recorded in the same run
(bench.py --copy-calib-mib: an elementwise int32 bitwise_not, N MiB read and written) to what the same counter reads for that copy.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def gemm_source_hash() -> str:
    """SHA-256 of the GEMM source with comments and blank space removed: a
    record stays valid across comment edits and goes stale on any code change."""
    with open(os.path.join(HERE, "csrc", "gemm.hip")) as f:
        src = f.read()
    code = []
    for line in src.splitlines():
        line = line.split("//", 1)[0].strip()
        if line:
            code.append(" ".join(line.split()))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()


def _per_kernel(path, counter):
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
    return out


def _pick(d, pred):
    vals = [v for k, vs in d.items() if pred(k) for v in vs]
    if not vals:
        raise SystemExit("kernel not found in counter file")
    return sum(vals) / len(vals)


def _per_dispatch(path, counter, name):
    """{(short kernel name, grid size): [bytes per dispatch, ...]} in dispatch order."""
    disp = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter or name not in r["Kernel_Name"]:
            continue
        short = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("nvfp4::", "")
        grid = r.get("Grid_Size_X", r.get("Grid_Size", ""))
        key = (short, grid, int(r["Dispatch_Id"]))
        disp[key] = disp.get(key, 0.0) + float(r["Counter_Value"]) * 1024.0
    out = {}
    for key in sorted(disp, key=lambda k: k[2]):
        out.setdefault(key[:2], []).append(disp[key])
    return out


def kernel_table(name, fetch_csv, write_csv, copy_mib) -> str:
    f_all = _per_kernel(fetch_csv, "FETCH_SIZE")
    w_all = _per_kernel(write_csv, "WRITE_SIZE")
    is_copy = lambda k: "bitwise_not" in k
    known = copy_mib * (1 << 20)
    fs, ws = known / _pick(f_all, is_copy), known / _pick(w_all, is_copy)
    f = _per_dispatch(fetch_csv, "FETCH_SIZE", name)
    w = _per_dispatch(write_csv, "WRITE_SIZE", name)
    mean = lambda v: sum(v[1:] or v) / len(v[1:] or v)
    rows = ["| Kernel | Grid | Fetch (MB) | Write (MB) |", "|---|---|---|---|"]
    for key in f:
        if key in w:
            rows.append("| `%s` | %s | %.2f | %.2f |" % (key[0], key[1], mean(f[key]) * fs / 1e6,
                                                       mean(w[key]) * ws / 1e6))
    rows.append("")
    rows.append("(fetch counts scaled by %.3f, writes by %.3f: the %d MiB copy's known bytes over its counts)"
                % (fs, ws, copy_mib))
    return "\n".join(rows)


def main(argv):
    if len(argv) > 1 and argv[1] == "--kernels":
        print(kernel_table(argv[2], argv[3], argv[4], int(argv[5])))
        return
    fetch_csv, write_csv, copy_mib, out_json = argv[1], argv[2], int(argv[3]), argv[4]
    f = _per_kernel(fetch_csv, "FETCH_SIZE")
    w = _per_kernel(write_csv, "WRITE_SIZE")
    is_fc1 = lambda k: "gemm_w4a4_kernel" in k and k.split("(")[0].rstrip(">").endswith("2")
    is_copy = lambda k: "bitwise_not" in k
    known = copy_mib * (1 << 20)
    copy_fetch, copy_write = _pick(f, is_copy), _pick(w, is_copy)
    fetch_scale, write_scale = known / copy_fetch, known / copy_write
    fc1_fetch, fc1_write = _pick(f, is_fc1), _pick(w, is_fc1)
    rec = {
        "workload": "qwen3_30b_a3b_moe_t8192",
        "gemm_source_sha256": gemm_source_hash(),
        "copy_known_bytes": known,
        "copy_fetch_counter_bytes": copy_fetch, "copy_write_counter_bytes": copy_write,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "fc1_fetch_bytes_raw": fc1_fetch, "fc1_write_bytes_raw": fc1_write,
        "fc1_hbm_bytes_per_launch": fc1_fetch * fetch_scale + fc1_write * write_scale,
    }
    with open(out_json, "w") as fo:
        json.dump(rec, fo, indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main(sys.argv)
