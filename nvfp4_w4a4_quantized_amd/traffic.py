"""HBM traffic of the FC1 kernel from two rocprofv3 counter passes.

Usage (after the two passes described in profiles/; run from the repository
root):
    python -m nvfp4_w4a4_quantized_amd.traffic FETCH_CSV WRITE_CSV COPY_MIB OUT_JSON

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


def main(argv):
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
