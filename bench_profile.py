#!/usr/bin/env python3
"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python bench_profile.py stats  <kernel_stats.csv> --cmd "<command>" --out profiles/X.txt
    python bench_profile.py traffic --gemm-fetch A.csv --gemm-write B.csv \
        --copy-fetch C.csv --copy-write D.csv --copy-bytes N --kernel tile_gemm \
        --cmd "<commands>" --out profiles/Y.md
    python bench_profile.py counters A.csv [B.csv ...] --kernel NAME --cmd "<commands>" \
        --out profiles/Z.md [--us MICROSECONDS]

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
CSRC = "dense_mixed_precision_02_amd/csrc"


def kernel_sources() -> list:
    """Every source the library is built from (kernels, path selection, the C ABI)."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(os.path.join(ROOT, CSRC))
                  if f.endswith((".hpp", ".hip", ".h")))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in kernel_sources():
        h.update(rel.encode())
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


def cmd_counters(a):
    """Per-dispatch medians of every counter in one or more --pmc CSVs for one
    kernel, plus the ratios they support (MI355X: 8 XCDs x 16 L2 channels,
    256 CUs, 1024 SIMDs; GRBM_GUI_ACTIVE summed over the XCDs)."""
    med = {}
    durs = []
    for path in a.csv:
        names = sorted({r["Counter_Name"] for r in csv.DictReader(open(path))})
        for n in names:
            v = per_dispatch(path, n, a.kernel)
            if v:
                med[n] = statistics.median(v[2:] or v)
        seen = {}
        for r in csv.DictReader(open(path)):
            if a.kernel in r["Kernel_Name"] and "Start_Timestamp" in r:
                seen[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        durs += [seen[k] for k in sorted(seen, key=int)][2:]
    us = a.us if a.us else (statistics.median(durs) if durs else None)
    lines = ["# rocprofv3 counters of one kernel launch (median over dispatches)", "",
             f"commands: {a.cmd}", f"kernel: {a.kernel}",
             f"kernel_source_sha256: {kernel_source_hash()}", ""]
    for n in sorted(med):
        lines.append(f"{n}: {med[n]:.6g}")
    g = med.get("GRBM_GUI_ACTIVE")
    if g:
        cyc = g / 8.0
        lines += ["", f"cycles per XCD (GRBM_GUI_ACTIVE / 8): {cyc:.0f}"]
        if us:
            lines.append(f"launch duration (median, counter runs): {us:.1f} us; "
                         f"effective clock {cyc / us / 1e3:.2f} GHz")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            lines.append(f"MFMA busy (per SIMD): {100 * med['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / cyc:.1f} %")
        if "TCC_BUSY_avr" in med:
            lines.append(f"L2 channel busy (TCC_BUSY_avr / cycles): {100 * med['TCC_BUSY_avr'] / cyc:.1f} %")
        if "TA_BUSY_avr" in med:
            lines.append(f"address unit busy (TA_BUSY_avr / cycles): {100 * med['TA_BUSY_avr'] / cyc:.1f} %")
        if "TCP_PENDING_STALL_CYCLES_sum" in med:
            lines.append(f"L1 stalled on pending L2 data: "
                         f"{100 * med['TCP_PENDING_STALL_CYCLES_sum'] / 256 / cyc:.1f} % of cycles per CU")
    if "SQ_LDS_IDX_ACTIVE" in med and med["SQ_LDS_IDX_ACTIVE"] > 0:
        act = med["SQ_LDS_IDX_ACTIVE"]
        for n, what in (("SQ_LDS_BANK_CONFLICT", "bank-conflict"), ("SQ_LDS_ADDR_CONFLICT", "address-conflict"),
                        ("SQ_LDS_UNALIGNED_STALL", "unaligned-stall"), ("SQ_LDS_DATA_FIFO_FULL", "data-FIFO-full")):
            if n in med:
                lines.append(f"LDS {what} cycles per LDS-active cycle ({n} / SQ_LDS_IDX_ACTIVE): "
                             f"{100 * med[n] / act:.2f} %")
    if "SQ_INSTS_LDS" in med and med.get("SQ_WAVES"):
        lines.append(f"LDS instructions per wave: {med['SQ_INSTS_LDS'] / med['SQ_WAVES']:.0f} "
                     f"({med['SQ_WAVES']:.0f} waves)")
    if "TCC_HIT_sum" in med and "TCC_MISS_sum" in med:
        h, m = med["TCC_HIT_sum"], med["TCC_MISS_sum"]
        lines.append(f"L2 hit rate: {100 * h / (h + m):.1f} %")
    if "TCP_TCC_READ_REQ_sum" in med:
        r = med["TCP_TCC_READ_REQ_sum"]
        lines.append(f"L1->L2 read requests: {r:.4g} (64 or 128 B each)")
        if "TCP_TCC_READ_REQ_LATENCY_sum" in med:
            lines.append(f"mean L2 read latency seen by L1: {med['TCP_TCC_READ_REQ_LATENCY_sum'] / r:.0f} cycles")
    text = "\n".join(lines) + "\n"
    open(a.out, "w").write(text)
    sys.stdout.write(text)


def cmd_ceiling(a):
    """The JSON lines of `bench.py --ceiling` as a table."""
    import json
    rows = [json.loads(x) for x in open(a.jsonl) if x.startswith("{")]
    lines = ["# Practical ceilings of this MI355X (tests/native/ceiling_probe.hip)", "",
             f"command: {a.cmd}", "",
             "Matrix instructions alone (independent accumulators, operands in registers,",
             "one workgroup of four waves per CU unless stated); rate = operations / launch time,",
             "median of the timed launches; clock = shader-clock counter ticks / launch time.", "",
             f"{'probe':<28} {'waves/SIMD':>10} {'rate':>10} {'unit':>8} {'of datasheet':>13} {'clock GHz':>10}"]
    for r in rows:
        if "frac_of_datasheet" in r:
            lines.append(f"{r['probe']:<28} {r['waves_per_simd']:>10} {r['rate']:>10.1f} {r['unit']:>8} "
                         f"{100 * r['frac_of_datasheet']:>12.1f}% {r['clock_counter_ghz']:>10.2f}")
    lines += ["", "Bandwidth (L2-resident 1 MB buffer swept by every workgroup; LDS; HBM streams of 2 GiB):", "",
              f"{'probe':<28} {'workgroups/CU':>13} {'rate':>10} {'unit':>6}"]
    for r in rows:
        if "frac_of_datasheet" not in r:
            wg = r.get("workgroups_per_cu", "")
            lines.append(f"{r['probe']:<28} {str(wg):>13} {r['rate']:>10.2f} {r['unit']:>6}")
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
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--us", type=float, default=None, help="launch duration, for the clock")
    e = sub.add_parser("ceiling")
    e.add_argument("jsonl")
    e.add_argument("--cmd", required=True)
    e.add_argument("--out", required=True)
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters,
     "ceiling": cmd_ceiling}[a.what](a)


if __name__ == "__main__":
    main()
