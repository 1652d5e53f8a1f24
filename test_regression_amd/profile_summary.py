"""Summarise rocprofv3 output for libmesa's kernels.

    python -m test_regression_amd.profile_summary stats <kernel_stats.csv | results.db> [--command CMD]
    python -m test_regression_amd.profile_summary traffic <fetch_counter_collection.csv>
        <write_counter_collection.csv> --copy-bytes N --kernel NAME_SUBSTRING [--first N] [--command CMD]

``stats`` prints per-kernel call counts and average durations (from a
``--kernel-trace --stats`` run, CSV or rocpd database).  ``traffic`` turns two
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs (KiB per dispatch) into HBM
bytes per launch of one kernel, each counter scaled by what it read for a
plain device copy of ``--copy-bytes`` bytes in the same run, and prints JSON
(with a hash of the CG kernel's source so stale numbers can be detected).

    python -m test_regression_amd.profile_summary mfma <counter_collection.csv> <agent_info.csv>
        --kernel NAME_SUBSTRING [--first N] [--command CMD] [--alg-flops F]

``mfma`` reads one ``--pmc`` run of SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE,
SQ_INSTS_VALU_MFMA_MOPS_F32, _BF16 and _F16 (any that were collected), SQ_INSTS_VALU,
SQ_INSTS_LDS, SQ_LDS_BANK_CONFLICT and SQ_LDS_IDX_ACTIVE and prints, per
dispatch of one kernel (median): the fraction of SIMD cycles the MFMA unit was
busy (busy cycles over GRBM_GUI_ACTIVE per XCD times the SIMD count, the
rocprofiler ``MfmaUtil`` definition with the per-XCD maximum taken as the sum
over XCDs divided by their count), the issued fp32 MFMA flops (512 per MOP),
the instruction mix, and the share of LDS cycles lost to bank conflicts.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sqlite3
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CG_SOURCES = ["test_regression_amd/csrc/cg_output.hip", "test_regression_amd/csrc/cg_output_bf16.hip",
              "test_regression_amd/csrc/cg_output_kernels.h", "test_regression_amd/csrc/cg_h2.h",
              "test_regression_amd/csrc/cg_core.h", "test_regression_amd/csrc/persistent.h",
              "test_regression_amd/csrc/mesa_device.h"]


def cg_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for p in sources or CG_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short(name: str) -> str:
    """Kernel name without its argument list."""
    return name.split("(")[0].replace("void ", "") if "(" in name else name


def read_stats(path: str):
    rows = []
    if path.endswith(".db"):
        c = sqlite3.connect(path)
        for name, calls, total, avg, pct in c.execute(
                "select name, total_calls, total_duration, average, percentage from top_kernels"):
            # the rocpd summary view is in microseconds already
            rows.append((short(name), int(calls), float(total), float(avg), float(pct)))
    else:
        for r in csv.DictReader(open(path)):
            rows.append((short(r["Name"]), int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
                         float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
    return rows


def cmd_stats(a):
    rows = read_stats(a.path)
    out = []
    if a.command:
        out.append(f"command: {a.command}")
    out.append(f"{'kernel':70s} {'calls':>6s} {'total_us':>12s} {'avg_us':>11s} {'pct':>6s}")
    for name, calls, tot, avg, pct in rows:
        if a.all or name.startswith("mesa::") or "zero_fill" in name:
            out.append(f"{name:70s} {calls:6d} {tot:12.1f} {avg:11.1f} {pct:6.2f}")
    if a.trace and a.first_kernel:
        # the first N dispatches of one kernel (one workload of a run that
        # launches the kernel for several), from the per-dispatch trace
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
             for r in csv.DictReader(open(a.trace)) if a.first_kernel in r["Kernel_Name"]][:a.first]
        if d:
            out.append(f"first {len(d)} dispatches of {a.first_kernel}: avg {statistics.mean(d):.1f} us, "
                       f"median {statistics.median(d):.1f} us")
        # without the first `skip` of them (a workload's untimed warmup launches)
        t = d[a.skip:]
        if a.skip and t:
            out.append(f"dispatches {a.skip + 1}..{len(d)} of {a.first_kernel}: avg {statistics.mean(t):.1f} us, "
                       f"median {statistics.median(t):.1f} us")
    print("\n".join(out))


def counter_rows(path: str, counter: str):
    res = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            res.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return res


def cmd_traffic(a):
    fetch = counter_rows(a.fetch, "FETCH_SIZE")
    write = counter_rows(a.write, "WRITE_SIZE")

    def copy_kib(rows):
        cands = [v for n, v in rows if "copyBuffer" in n or "copy" in n.lower()]
        return max(cands) if cands else None

    copy_gib = a.copy_bytes / 2 ** 30
    f_copy, w_copy = copy_kib(fetch), copy_kib(write)
    f_scale = a.copy_bytes / 1024 / f_copy
    w_scale = a.copy_bytes / 1024 / w_copy
    f_k = [v for n, v in fetch if a.kernel in n]
    w_k = [v for n, v in write if a.kernel in n]
    if a.first:
        # only the first dispatches (one workload of a run that launches the
        # same kernel for several)
        f_k, w_k = f_k[:a.first], w_k[:a.first]
    fb = statistics.median(f_k) * 1024 * f_scale
    wb = statistics.median(w_k) * 1024 * w_scale
    print(json.dumps({
        "kernel": a.kernel, "command": a.command, "kernel_source_hash": cg_source_hash(a.sources),
        "sources": a.sources or CG_SOURCES,
        "fetch_kib_per_dispatch": statistics.median(f_k), "write_kib_per_dispatch": statistics.median(w_k),
        "copy_probe_bytes": a.copy_bytes, "copy_probe_gib": copy_gib,
        "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
        "bytes_per_launch": round(fb + wb), "dispatches": [len(f_k), len(w_k)], "first": a.first,
    }, indent=1))


def cmd_mfma(a):
    per = {}
    for r in csv.DictReader(open(a.counters)):
        if a.kernel not in r["Kernel_Name"]:
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), {
            "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    agent = next(r for r in csv.DictReader(open(a.agents)) if r.get("Name", "").startswith("gfx"))
    nxcc, nsimd = int(agent["Num_Xcc"]), int(agent["Simd_Count"])
    disp = [per[k] for k in sorted(per)]
    if a.first:
        disp = disp[:a.first]
    med = lambda f: statistics.median(f(d) for d in disp)
    cycles = med(lambda d: d["GRBM_GUI_ACTIVE"] / nxcc)
    mops = med(lambda d: d.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0))
    mops_bf = med(lambda d: d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0))
    mops_h = med(lambda d: d.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0))
    ns = med(lambda d: d["ns"])
    out = {
        "kernel": a.kernel, "command": a.command, "kernel_source_hash": cg_source_hash(a.sources),
        "sources": a.sources or CG_SOURCES, "dispatches": len(disp), "first": a.first,
        "gpu": agent["Name"], "xcc": nxcc, "simds": nsimd,
        "duration_us_under_counters": round(ns / 1e3, 1),
        "clock_mhz": round(cycles / ns * 1e3, 1),
        "mfma_busy_frac": round(med(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / nxcc * nsimd)), 4),
        "mfma_f32_issued_flops": mops * 512,
        "mfma_bf16_issued_flops": mops_bf * 512,
        "mfma_f16_issued_flops": mops_h * 512,
        "valu_instructions": med(lambda d: d["SQ_INSTS_VALU"]),
        "lds_instructions": med(lambda d: d["SQ_INSTS_LDS"]),
        "lds_bank_conflict_frac": round(med(lambda d: d["SQ_LDS_BANK_CONFLICT"] / d["SQ_LDS_IDX_ACTIVE"]
                                            if d["SQ_LDS_IDX_ACTIVE"] else 0.0), 4),
    }
    if a.alg_flops:
        out["algorithmic_flops"] = a.alg_flops
        out["issued_mfma_over_algorithmic"] = round((mops + mops_bf + mops_h) * 512 / a.alg_flops, 4)
    print(json.dumps(out, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("path")
    s.add_argument("--command", default="")
    s.add_argument("--all", action="store_true")
    s.add_argument("--trace", default="", help="kernel_trace.csv of the same run")
    s.add_argument("--first-kernel", default="", help="kernel name substring for --first")
    s.add_argument("--first", type=int, default=0, help="average only its first N dispatches")
    s.add_argument("--skip", type=int, default=0, help="also average those first N without their first SKIP")
    t = sub.add_parser("traffic")
    t.add_argument("fetch")
    t.add_argument("write")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--command", default="")
    t.add_argument("--first", type=int, default=0,
                   help="use only the first N matching dispatches (0: all)")
    t.add_argument("--sources", nargs="*", default=None,
                   help="repository-relative sources whose hash identifies the kernel (default: the CG kernel's)")
    m = sub.add_parser("mfma")
    m.add_argument("counters")
    m.add_argument("agents")
    m.add_argument("--kernel", required=True)
    m.add_argument("--command", default="")
    m.add_argument("--first", type=int, default=0)
    m.add_argument("--alg-flops", type=float, default=0.0, help="algorithmic flops per launch")
    m.add_argument("--sources", nargs="*", default=None)
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "mfma": cmd_mfma}[a.what](a)


if __name__ == "__main__":
    sys.exit(main())
