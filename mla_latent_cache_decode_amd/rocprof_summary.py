"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

Two modes:

  stats    from a ``rocprofv3 --kernel-trace --stats --output-format csv`` run:
           per-kernel call count and average / min / max duration over all
           calls, and (with --last N) the average over each kernel's last N
           dispatches from the kernel trace: the timed steps of a bench run,
           after its warm-up.
  counters from one or more ``rocprofv3 --pmc`` runs: per-dispatch averages
           of each counter of one kernel, and derived figures (the clock the
           dispatches ran at, matrix-core busy fraction, MFMA rate, LDS bank
           conflicts per LDS-active cycle).
  traffic  from two ``rocprofv3 --pmc`` runs (FETCH_SIZE, then WRITE_SIZE;
           both in KiB per dispatch) of ``bench.py --copy-mb N``: the HBM
           bytes per dispatch of one kernel, each counter scaled by what it
           reads for the plain N MiB device copy in the same run (which moves
           exactly N MiB each way).  The summary records a hash of the
           kernel's source files; bench.py reports the traffic only while
           that hash still matches.

Usage:
  python -m mla_latent_cache_decode_amd.rocprof_summary stats --csv DIR/run_kernel_stats.csv \\
      --command "..." --out profiles/x.txt
  python -m mla_latent_cache_decode_amd.rocprof_summary traffic --fetch F.csv --write W.csv \\
      --kernel mla_decode_bf16_kernel --copy-mb 1024 --command-fetch "..." --command-write "..." --out profiles/y.txt
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
# the source files each decode kernel is built from
KERNEL_SOURCES = {
    "mla_decode_bf16_kernel": ("csrc/decode_bf16.hip", "csrc/decode_common.h", "csrc/mla_internal.h"),
    "mla_decode_kernel": ("csrc/decode.hip", "csrc/decode_rowsplit.h", "csrc/decode_common.h", "csrc/mla_internal.h"),
    "mla_decode_mx_kernel": ("csrc/decode_mx.hip", "csrc/decode_rowsplit.h", "csrc/decode_common.h",
                             "csrc/mla_internal.h"),
}


def kernel_for_dtype(kv_dtype: str, sparse: bool = False) -> str:
    """Name of the decode kernel that serves a cache dtype (the dense and the
    sparse decode of one dtype share their kernel)."""
    if kv_dtype == "bf16":
        return "mla_decode_bf16_kernel"
    return "mla_decode_mx_kernel" if kv_dtype == "fp8" else "mla_decode_kernel"


def _code_only(text: str) -> str:
    """Source text without comments and blank lines (comment edits do not
    change the kernel; a string literal holding // is not expected here)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", l).rstrip() for l in text.splitlines()]
    return "\n".join(l for l in lines if l.strip())


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code (comments stripped) a decode kernel is built from."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(PKG, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(path: str) -> dict | None:
    """Parse a traffic summary written by this module; None if absent/unparsable."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    try:
        return {"source_hash": vals["source_hash"], "bytes_per_launch": int(vals["hbm_bytes_per_launch"]),
                "read_bytes": int(vals["read_bytes_per_launch"]),
                "write_bytes": int(vals["write_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None


def _short(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0][:60]


def _stats(args) -> str:
    rows = list(csv.DictReader(open(args.csv)))
    lines = [f"command: {args.command}", "", "all calls:",
             f"{'kernel':<60} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    for r in rows:
        lines.append(f"{_short(r['Name']):<60} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                     f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
                     f"{float(r['Percentage']):>6.2f}")
    if args.last:
        trace = os.path.join(os.path.dirname(args.csv), os.path.basename(args.csv).replace("kernel_stats", "kernel_trace"))
        per: dict[str, list[float]] = {}
        for r in csv.DictReader(open(trace)):
            per.setdefault(r["Kernel_Name"], []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        skip = args.skip_last
        what = f"dispatches -{args.last + skip} .. -{skip + 1} of each kernel" if skip else \
            f"last {args.last} dispatches of each kernel"
        lines += ["", f"{what} ({args.label}):",
                  f"{'kernel':<60} {'n':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}"]
        for name, ds in per.items():
            if len(ds) < args.last + skip:
                continue
            d = ds[len(ds) - skip - args.last:len(ds) - skip]
            lines.append(f"{_short(name):<60} {len(d):>6} {statistics.mean(d):>10.2f} {min(d):>10.2f} {max(d):>10.2f}")
    return "\n".join(lines) + "\n"


def _per_kernel(path: str, counter: str) -> dict:
    out: dict[str, list[tuple[int, float]]] = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def _traffic(args) -> str:
    copy_bytes = args.copy_mb * (1 << 20)
    res = {}
    for tag, path, counter in (("read", args.fetch, "FETCH_SIZE"), ("write", args.write, "WRITE_SIZE")):
        pk = _per_kernel(path, counter)
        copies = [v for k, vs in pk.items() if "copyBuffer" in k for v in vs]
        if not copies:
            sys.exit(f"no copy kernel in {path}")
        _, copy_kib = max(copies)                       # the big calibration copy
        factor = copy_bytes / (copy_kib * 1024.0)
        mine = [v for k, vs in pk.items() if _short(k).split("<")[0].split("::")[-1] == args.kernel for _, v in vs]
        if not mine:
            sys.exit(f"no {args.kernel} dispatch in {path}")
        kib = statistics.mean(mine)
        res[tag] = (kib, factor, len(mine), copy_kib)
    rb = int(round(res["read"][0] * 1024 * res["read"][1]))
    wb = int(round(res["write"][0] * 1024 * res["write"][1]))
    lines = [
        f"kernel: {args.kernel}",
        f"workload: {args.workload}",
        f"source_hash: {kernel_source_hash(args.kernel)}",
        f"read_bytes_per_launch: {rb}",
        f"write_bytes_per_launch: {wb}",
        f"hbm_bytes_per_launch: {rb + wb}",
        "",
        f"FETCH_SIZE: {res['read'][0]:.1f} KiB/dispatch over {res['read'][2]} dispatches; "
        f"the {args.copy_mb} MiB copy read {res['read'][3]:.1f} KiB -> factor {res['read'][1]:.4f}",
        f"WRITE_SIZE: {res['write'][0]:.1f} KiB/dispatch over {res['write'][2]} dispatches; "
        f"the {args.copy_mb} MiB copy wrote {res['write'][3]:.1f} KiB -> factor {res['write'][1]:.4f}",
        "",
        f"command (fetch): {args.command_fetch}",
        f"command (write): {args.command_write}",
    ]
    return "\n".join(lines) + "\n"


def _counters(args) -> str:
    """Per-dispatch averages of every counter of one kernel over one or more
    ``--pmc`` runs (one CSV each), plus the clock the dispatches ran at when
    GRBM_GUI_ACTIVE (GPU clock cycles) and the dispatch timestamps are there."""
    lines = [f"kernel: {args.kernel}", f"workload: {args.workload}",
             f"source_hash: {kernel_source_hash(args.kernel) if args.kernel in KERNEL_SOURCES else '-'}", ""]
    vals: dict[str, float] = {}
    for path, cmd in zip(args.csv, args.command):
        per: dict[str, list[float]] = {}
        dur_by_dispatch: dict[str, int] = {}
        for r in csv.DictReader(open(path)):
            if _short(r["Kernel_Name"]).split("<")[0].split("::")[-1] != args.kernel:
                continue
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                dur_by_dispatch[r.get("Dispatch_Id", str(len(dur_by_dispatch)))] = \
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        durs = list(dur_by_dispatch.values())
        if not per:
            sys.exit(f"no {args.kernel} dispatch in {path}")
        n = min(len(v) for v in per.values())
        last = args.last or n
        lines.append(f"command: {cmd}")
        lines.append(f"  dispatches: {n} (averaged over the last {min(last, n)})")
        for name in sorted(per):
            v = statistics.mean(per[name][-last:])
            vals[name] = v
            lines.append(f"  {name:<36} {v:>20.1f}")
        if durs:
            d = statistics.mean(durs[-last:])
            vals["_duration_ns"] = d
            lines.append(f"  {'dispatch duration (ns)':<36} {d:>20.1f}")
        lines.append("")
    lines.append("derived (GRBM_GUI_ACTIVE counts GPU clock cycles summed over the XCDs):")
    if "GRBM_GUI_ACTIVE" in vals and "_duration_ns" in vals:
        cyc = vals["GRBM_GUI_ACTIVE"] / args.xcds
        lines.append(f"  GPU clock over the dispatch = GRBM_GUI_ACTIVE / {args.xcds} / duration = "
                     f"{cyc / vals['_duration_ns'] * 1e3:.0f} MHz")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "GRBM_GUI_ACTIVE" in vals:
        simd_cycles = vals["GRBM_GUI_ACTIVE"] / args.xcds * args.cus * 4
        lines.append(f"  matrix cores busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {args.xcds} x {args.cus} CUs "
                     f"x 4 SIMDs) = {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.3f}")
    kinds = [k for k in ("BF16", "F16", "F8", "F6F4") if f"SQ_INSTS_VALU_MFMA_MOPS_{k}" in vals]
    mops = sum(vals[f"SQ_INSTS_VALU_MFMA_MOPS_{k}"] for k in kinds)
    if mops and "_duration_ns" in vals:
        lines.append(f"  MFMA work = ({' + '.join('MOPS_' + k for k in kinds)}) x 512 flop = {mops * 512 / 1e9:.2f} "
                     f"GFLOP per dispatch; over the dispatch duration {mops * 512 / vals['_duration_ns'] / 1e3:.1f} TFLOP/s")
    if "SQ_LDS_BANK_CONFLICT" in vals and "SQ_LDS_IDX_ACTIVE" in vals and vals["SQ_LDS_IDX_ACTIVE"]:
        lines.append(f"  LDS bank-conflict cycles / LDS active cycles = "
                     f"{vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_LDS_IDX_ACTIVE']:.4f}")
    if "TCP_TCC_READ_REQ_LATENCY" in vals and vals.get("TCP_TCC_READ_REQ"):
        lines.append(f"  mean L1 -> L2 read latency = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ = "
                     f"{vals['TCP_TCC_READ_REQ_LATENCY'] / vals['TCP_TCC_READ_REQ']:.0f} cycles")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--last", type=int, default=0, help="also average the last N dispatches per kernel")
    s.add_argument("--skip-last", type=int, default=0, help="... leaving out the final M dispatches")
    s.add_argument("--label", default="the timed steps")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-mb", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", required=True, action="append", help="one per --pmc run")
    c.add_argument("--command", required=True, action="append", help="one per --pmc run, same order")
    c.add_argument("--kernel", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--last", type=int, default=0, help="average the last N dispatches (0: all)")
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    text = {"stats": _stats, "traffic": _traffic, "counters": _counters}[args.mode](args)
    with open(args.out, "w") as f:
        f.write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
