"""Summaries of rocprofv3 output for the kernels of this library.

Two commands, both reading the CSV files that ``rocprofv3 --output-format csv``
writes:

    python -m adaptive_sparse_attention_amd.profiling stats RUN_kernel_stats.csv \
        --command "..." --out profiles/<name>.txt
    python -m adaptive_sparse_attention_amd.profiling traffic \
        --fetch FETCH/run_counter_collection.csv --write WRITE/run_counter_collection.csv \
        --copy-bytes B --command "..." --out profiles/<name>.txt --json profiles/traffic.json

    python -m adaptive_sparse_attention_amd.profiling counters A/run_counter_collection.csv \
        B/run_counter_collection.csv --command "..." --out profiles/<name>.txt

``counters`` averages every counter of one or more counter-collection runs
per kernel and derives: MFMA utilisation (SQ_VALU_MFMA_BUSY_CYCLES, summed
over the SIMDs, over the SIMD cycles of the dispatch at the 2.4 GHz peak
clock: 1024 SIMDs x 2.4 cycles/ns x its End - Start timestamps), MFMA FLOPs
(512 per
SQ_INSTS_VALU_MFMA_MOPS_* op), other VALU and SALU instructions per MFMA
instruction, the waiting fraction SQ_WAIT_ANY / SQ_WAVE_CYCLES, and LDS bank
conflict cycles per LDS instruction and per active LDS cycle.

``traffic`` turns the per-dispatch FETCH_SIZE and WRITE_SIZE counters (KiB)
into bytes per launch. Each counter is first scaled by what it reads for a
plain elementwise copy of known size in the same run (a kernel that reads and
writes exactly ``copy_bytes`` each), so that the figure is in the same units
as the algorithmic byte counts. The JSON records the hash of the kernel
sources, so a stale figure is not reported after the kernels change.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("ea_common.hpp", "ea_fwd.hpp", "ea_bwd.hpp", "ea_launch_impl.hpp", "k_mask.hip")
COPY_MARKER = "neg"      # torch.neg is the calibration copy (one read, one write per element)


def kernel_source_sha() -> str:
    """Hash of the kernel sources: identifies the kernels a counter figure belongs to."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(_HERE, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    """'void ea::fwd_out_kernel<ea::BF16, 64, 1, 2>(ea::FwdArgs)' -> 'fwd_out_kernel<BF16, 64, 1, 2>'."""
    s = name.split("(")[0]
    for p in ("void ", "ea::"):
        s = s.replace(p, "")
    return s.strip()


def base_name(name: str) -> str:
    return short_name(name).split("<")[0]


def read_csv(path: str):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def stats_table(path: str):
    """Rows of a kernel_stats.csv as (name, calls, avg_ms, total_ms, percent)."""
    out = []
    for r in read_csv(path):
        out.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) * 1e-6,
                    float(r["TotalDurationNs"]) * 1e-6, float(r["Percentage"])))
    out.sort(key=lambda t: -t[3])
    return out


def counter_avgs(path: str, counter: str):
    """Average of `counter` per dispatch, by kernel name."""
    acc = collections.defaultdict(list)
    for r in read_csv(path):
        if r["Counter_Name"] != counter:
            continue
        acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


CUS, SIMDS, PEAK_GHZ = 256, 4, 2.4


def counter_table(paths):
    """{kernel: {counter: average per dispatch}} over the given CSV files;
    "DURATION_NS" holds the average End - Start timestamp of its dispatches."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for i, path in enumerate(paths):
        for r in read_csv(path):
            acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                dur[r["Kernel_Name"]][(i, r["Dispatch_Id"])] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    out = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}
    for k, d in dur.items():
        if d:
            out[k]["DURATION_NS"] = sum(d.values()) / len(d)
    return out


def derived(c: dict) -> dict:
    """Derived metrics of one kernel's averaged counters (missing inputs skipped)."""
    out = {}
    t = c.get("DURATION_NS")
    if t and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        out["mfma_util"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (CUS * SIMDS * PEAK_GHZ * t)
    mops = sum(v for n, v in c.items() if n.startswith("SQ_INSTS_VALU_MFMA_MOPS_"))
    if any(n.startswith("SQ_INSTS_VALU_MFMA_MOPS_") for n in c):
        out["mfma_flop"] = 512.0 * mops
    m = c.get("SQ_INSTS_MFMA")
    if m:
        if "SQ_INSTS_VALU" in c:
            out["valu_per_mfma"] = (c["SQ_INSTS_VALU"] - m) / m
        if "SQ_INSTS_SALU" in c:
            out["salu_per_mfma"] = c["SQ_INSTS_SALU"] / m
    if c.get("SQ_WAVE_CYCLES") and "SQ_WAIT_ANY" in c:
        out["wait_frac"] = c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]
    if c.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in c:
        out["lds_conflict_per_inst"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_INSTS_LDS"]
    if c.get("SQ_ACTIVE_INST_LDS") and "SQ_LDS_BANK_CONFLICT" in c:
        out["lds_conflict_frac"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_ACTIVE_INST_LDS"]
    return out


def cmd_counters(args) -> int:
    tab = counter_table(args.csv)
    cols = [("mfma_util", "MFMA util", "{:.3f}"), ("mfma_flop", "MFMA GFLOP", "{:.1f}"),
            ("valu_per_mfma", "VALU/MFMA", "{:.2f}"), ("salu_per_mfma", "SALU/MFMA", "{:.2f}"),
            ("wait_frac", "wait", "{:.3f}"), ("lds_conflict_per_inst", "LDS cfl/inst", "{:.3f}"),
            ("lds_conflict_frac", "LDS cfl/act", "{:.3f}")]
    lines = [f"# rocprofv3 counters: {args.title}", "", "Commands (one counter set per run):", "",
             f"    {args.command}", "",
             "MFMA util = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x 2.4 cycles/ns x dispatch duration); "
             "MFMA GFLOP = 512 x SQ_INSTS_VALU_MFMA_MOPS_* / 1e9 per dispatch;",
             "VALU/MFMA = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA; SALU/MFMA = SQ_INSTS_SALU / "
             "SQ_INSTS_MFMA; wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES;",
             "LDS cfl/inst = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS; LDS cfl/act = SQ_LDS_BANK_CONFLICT / "
             "SQ_ACTIVE_INST_LDS. Averages per dispatch.", "",
             f"{'kernel':44s} " + " ".join(f"{h:>12s}" for _, h, _ in cols)]
    rows = []
    for k, c in tab.items():
        if "ea::" not in k:
            continue
        d = derived(c)
        if "mfma_flop" in d:
            d["mfma_flop"] /= 1e9
        rows.append((c.get("DURATION_NS", 0.0), short_name(k), d))
    for _, n, d in sorted(rows, key=lambda t: -t[0]):
        lines.append(f"{n[:44]:44s} " + " ".join(
            f"{(fmt.format(d[key]) if key in d else '-'):>12s}" for key, _, fmt in cols))
    _write(args.out, "\n".join(lines) + "\n")
    return 0


def cmd_stats(args) -> int:
    rows = stats_table(args.csv)
    lines = [f"# rocprofv3 kernel statistics: {args.title}", "",
             "Command:", "", f"    {args.command}", "",
             f"{'kernel':64s} {'calls':>6s} {'avg ms':>10s} {'total ms':>10s} {'%':>6s}"]
    for n, c, a, t, p in rows:
        lines.append(f"{n[:64]:64s} {c:6d} {a:10.4f} {t:10.3f} {p:6.2f}")
    text = "\n".join(lines) + "\n"
    _write(args.out, text)
    return 0


def cmd_traffic(args) -> int:
    fetch = counter_avgs(args.fetch, "FETCH_SIZE")
    write = counter_avgs(args.write, "WRITE_SIZE")
    copy_f = [v for k, v in fetch.items() if COPY_MARKER in k.lower()]
    copy_w = [v for k, v in write.items() if COPY_MARKER in k.lower()]
    if not copy_f or not copy_w:
        print("no calibration copy kernel in the counter files", file=sys.stderr)
        return 1
    # counters are in KiB per dispatch; factor = true bytes / counted bytes
    f_fetch = args.copy_bytes / (copy_f[0][0] * 1024.0)
    f_write = args.copy_bytes / (copy_w[0][0] * 1024.0)
    sha = kernel_source_sha()
    rec = {"_calibration": {"copy_bytes": args.copy_bytes, "fetch_kib": copy_f[0][0], "write_kib": copy_w[0][0],
                            "fetch_factor": f_fetch, "write_factor": f_write, "command": args.command}}
    lines = [f"# HBM traffic per launch (FETCH_SIZE, WRITE_SIZE): {args.title}", "",
             "Commands (one counter per run):", "", f"    {args.command}", "",
             f"Calibration: torch.neg over {args.copy_bytes} bytes reads {copy_f[0][0]:.0f} KiB "
             f"(factor {f_fetch:.4f}) and writes {copy_w[0][0]:.0f} KiB (factor {f_write:.4f}).", "",
             f"{'kernel':52s} {'n':>3s} {'fetch MB':>10s} {'write MB':>10s} {'total MB':>10s}"]
    for k in sorted(fetch, key=lambda k: -fetch[k][0]):
        if "ea::" not in k:
            continue
        fb = fetch[k][0] * 1024.0 * f_fetch
        wb = write.get(k, (0.0, 0))[0] * 1024.0 * f_write
        name = base_name(k)
        rec[name] = {"kernel": short_name(k), "fetch_bytes": fb, "write_bytes": wb,
                     "traffic_bytes_per_launch": fb + wb, "dispatches": fetch[k][1], "source_sha": sha}
        lines.append(f"{short_name(k)[:52]:52s} {fetch[k][1]:3d} {fb / 1e6:10.2f} {wb / 1e6:10.2f} "
                     f"{(fb + wb) / 1e6:10.2f}")
    lines += ["", f"kernel source hash: {sha}"]
    _write(args.out, "\n".join(lines) + "\n")
    if args.json:
        with open(args.json, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
            f.write("\n")
    return 0


def _write(path, text):
    if path:
        with open(path, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--out")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="")
    t.add_argument("--out")
    t.add_argument("--json")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--command", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--out")
    args = ap.parse_args(argv)
    return {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
