#!/usr/bin/env python3
"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python bench_profile.py stats  <kernel_stats.csv> --cmd "<command>" --out profiles/X.txt
    python bench_profile.py traffic --gemm-fetch A.csv --gemm-write B.csv \
        --copy-fetch C.csv --copy-write D.csv --copy-bytes N --kernel tile_gemm \
        --cmd "<commands>" --out profiles/Y.md

The traffic summary scales the per-dispatch FETCH_SIZE / WRITE_SIZE of the GEMM
kernel by the ratio (known bytes / counter bytes) that the same counters show
for a plain device-to-device copy of known size, and records a hash of the
kernel sources so that bench.py can tell when the figures are stale.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["dense_mixed_precision_02_amd/csrc/common.hpp",
                  "dense_mixed_precision_02_amd/csrc/tile_gemm.hpp",
                  "dense_mixed_precision_02_amd/csrc/aux_kernels.hpp",
                  "dense_mixed_precision_02_amd/csrc/gemm_api.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def per_dispatch(csv_path: str, counter: str, name_part: str):
    """Per-dispatch values of one counter for kernels whose name contains name_part
    (summed over the counter's instances, e.g. over XCDs)."""
    vals = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or name_part not in r["Kernel_Name"]:
                continue
            key = r["Dispatch_Id"]
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return [vals[k] for k in sorted(vals, key=int)]


def cmd_stats(a):
    rows = list(csv.DictReader(open(a.csv)))
    out = [f"# rocprofv3 kernel statistics", f"command: {a.cmd}", "",
           f"{'kernel':<72} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    for r in rows:
        name = r["Name"][:72]
        calls = int(r["Calls"])
        avg = float(r["AverageNs"]) / 1e3
        mn = float(r["MinNs"]) / 1e3
        mx = float(r["MaxNs"]) / 1e3
        pct = float(r["Percentage"])
        out.append(f"{name:<72} {calls:>6} {avg:>10.2f} {mn:>10.2f} {mx:>10.2f} {pct:>6.2f}")
    text = "\n".join(out) + "\n"
    open(a.out, "w").write(text)
    sys.stdout.write(text)


def cmd_traffic(a):
    gf = per_dispatch(a.gemm_fetch, "FETCH_SIZE", a.kernel)
    gw = per_dispatch(a.gemm_write, "WRITE_SIZE", a.kernel)
    cf = per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw = per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    if not (gf and gw and cf and cw):
        raise SystemExit("missing dispatches for a counter")
    kib = 1024.0
    # skip the first dispatches (warm-up / first touch)
    g_fetch = statistics.median(gf[2:] or gf) * kib
    g_write = statistics.median(gw[2:] or gw) * kib
    c_fetch = statistics.median(cf[1:] or cf) * kib
    c_write = statistics.median(cw[1:] or cw) * kib
    f_scale = a.copy_bytes / c_fetch
    w_scale = a.copy_bytes / c_write
    fetch = g_fetch * f_scale
    write = g_write * w_scale
    lines = [
        "# HBM traffic of one GEMM launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)",
        "",
        f"commands: {a.cmd}",
        f"kernel: {a.kernel}",
        f"kernel_source_sha256: {kernel_source_hash()}",
        "",
        f"gemm FETCH_SIZE per dispatch (median): {g_fetch / kib:.1f} KiB ({len(gf)} dispatches)",
        f"gemm WRITE_SIZE per dispatch (median): {g_write / kib:.1f} KiB ({len(gw)} dispatches)",
        f"copy kernel ({a.copy_kernel}) of {a.copy_bytes} bytes: FETCH_SIZE {c_fetch / kib:.1f} KiB, "
        f"WRITE_SIZE {c_write / kib:.1f} KiB",
        f"calibration factors (known bytes / counter bytes): fetch {f_scale:.4f}, write {w_scale:.4f}",
        "",
        f"fetch_bytes_per_launch: {fetch:.0f}",
        f"write_bytes_per_launch: {write:.0f}",
        f"traffic_bytes_per_launch: {fetch + write:.0f}",
    ]
    text = "\n".join(lines) + "\n"
    open(a.out, "w").write(text)
    sys.stdout.write(text)


def read_traffic(path: str):
    """(bytes per launch, source hash) from a traffic summary, or None."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    try:
        return float(vals["traffic_bytes_per_launch"]), vals["kernel_source_sha256"]
    except KeyError:
        return None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for k in ("gemm-fetch", "gemm-write", "copy-fetch", "copy-write", "cmd", "out"):
        t.add_argument("--" + k, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--kernel", default="tile_gemm")
    t.add_argument("--copy-kernel", default="copyBuffer")
    a = ap.parse_args()
    (cmd_stats if a.what == "stats" else cmd_traffic)(a)


if __name__ == "__main__":
    main()
