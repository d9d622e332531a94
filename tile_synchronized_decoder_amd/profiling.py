"""Summaries of rocprofv3 output for the profiles kept beside the code.

    python -m tile_synchronized_decoder_amd.profiling stats RUN_kernel_stats.csv --command "..."
    python -m tile_synchronized_decoder_amd.profiling traffic FETCH_counter_collection.csv \
        WRITE_counter_collection.csv --kernel mk_interp --copy-mib 1024 --algorithmic BYTES --command "..."

    python -m tile_synchronized_decoder_amd.profiling mfma RUN_counter_collection.csv \
        --kernel mk_interp_prefill --flops FLOPS --command "..."

`traffic` turns the FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch) of
one kernel into HBM bytes per launch.  Each counter is scaled by what it reads
for a plain device copy of known size in the same run (rocclr's copyBuffer
reads the source once; torch's fill writes the destination once), so request
sizes the derived counter does not weigh correctly cancel out.  The summary
records a hash of the kernel sources; a reader of the summary treats the
figure as stale once the sources have changed.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
from typing import Dict, List, Optional

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
KERNEL_SOURCES = ("kernels.h", "inst.hip", "api.hip")


def kernel_sources_sha() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stats_markdown(path: str, command: str, top: int = 24) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["# Kernel time summary", "", "Command:", "", "```", command, "```", "",
           "| kernel | calls | avg (us) | min (us) | max (us) | total % |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        n = r["Name"].replace("|", "/")
        if len(n) > 90:
            n = n[:87] + "..."
        out.append(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f} |")
    return "\n".join(out) + "\n"


def _per_kernel(path: str, counter: str) -> Dict[str, List[float]]:
    agg: Dict[str, List[float]] = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            agg.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return agg


def _largest(agg: Dict[str, List[float]], key: str) -> Optional[float]:
    vals = [v for name, vs in agg.items() if key in name for v in vs]
    return max(vals) if vals else None


def _median(agg: Dict[str, List[float]], key: str) -> Optional[float]:
    vals = [v for name, vs in agg.items() if key in name for v in vs]
    return statistics.median(vals) if vals else None


def traffic_markdown(fetch_csv: str, write_csv: str, kernel: str, copy_mib: int, algorithmic: int,
                     command: str) -> str:
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    f_copy = _largest(fetch, "copyBuffer")            # the copy reads copy_mib MiB
    w_fill = _largest(write, "FillFunctor")           # torch.ones writes copy_mib MiB
    f_k, w_k = _median(fetch, kernel), _median(write, kernel)
    fs = copy_kib / f_copy if f_copy else None
    wsc = copy_kib / w_fill if w_fill else None
    traffic = (f_k * fs + w_k * wsc) * 1024.0 if None not in (f_k, w_k, fs, wsc) else None
    lines = ["# HBM traffic per launch from hardware counters", "",
             "Commands (one counter per run):", "", "```", command, "```", "",
             f"Calibration: a {copy_mib} MiB device copy reads FETCH_SIZE = {f_copy:.0f} KiB "
             f"(scale {fs:.4f}); a {copy_mib} MiB fill writes WRITE_SIZE = {w_fill:.0f} KiB (scale {wsc:.4f}).", "",
             "| kernel | dispatches | FETCH_SIZE KiB (median) | WRITE_SIZE KiB (median) | scaled bytes |",
             "|---|---|---|---|---|"]
    for name in sorted(set(fetch) | set(write), key=lambda n: -(_median(fetch, n) or 0)):
        fm, wm = _median(fetch, name), _median(write, name)
        if not fm and not wm:
            continue
        sb = ((fm or 0) * (fs or 0) + (wm or 0) * (wsc or 0)) * 1024.0
        short = name.replace("|", "/")
        short = short if len(short) <= 80 else short[:77] + "..."
        lines.append(f"| `{short}` | {len(fetch.get(name, []))} | {fm or 0:.0f} | {wm or 0:.0f} | {sb:.4g} |")
    lines += ["", f"Kernel `{kernel}`: algorithmic bytes per launch {algorithmic}; counted traffic "
              f"{traffic:.6g} bytes ({traffic / algorithmic:.4f} x algorithmic).", "",
              f"traffic_bytes_per_launch: {int(round(traffic))}",
              f"algorithmic_bytes_per_launch: {algorithmic}",
              f"kernel_sources_sha256: {kernel_sources_sha()}", ""]
    return "\n".join(lines)


def mfma_markdown(pmc_csv: str, kernel: str, flops: int, command: str) -> str:
    """Matrix-core evidence for the kernels of one --pmc run that collected the
    derived counters MfmaUtil (busy cycles of the MFMA units over all SIMDs and
    the GPU's active cycles) and MfmaFlopsBF16 (bf16 MFMA operations)."""
    util = _per_kernel(pmc_csv, "MfmaUtil")
    fl = _per_kernel(pmc_csv, "MfmaFlopsBF16")
    lines = ["# Matrix-core use per dispatch from hardware counters", "",
             "Command:", "", "```", command, "```", "",
             "| kernel | dispatches | MfmaUtil % (median) | bf16 MFMA FLOP per dispatch (median) |",
             "|---|---|---|---|"]
    for name in sorted(set(util) | set(fl), key=lambda n: -(_median(fl, n) or 0)):
        u, f = _median(util, name), _median(fl, name)
        if not f:
            continue
        short = name.replace("|", "/")
        short = short if len(short) <= 80 else short[:77] + "..."
        lines.append(f"| `{short}` | {len(fl.get(name, []))} | {u or 0:.1f} | {f:.4g} |")
    f_k, u_k = _median(fl, kernel), _median(util, kernel)
    if f_k:
        lines += ["", f"Kernel `{kernel}`: algorithmic matrix FLOP per launch {flops}; the counters count "
                  f"{f_k:.6g} ({f_k / flops:.4f} x algorithmic); MFMA units busy {u_k:.1f}% of the active cycles.",
                  "", f"mfma_util_percent: {u_k:.2f}", f"mfma_flops_per_launch: {int(round(f_k))}",
                  f"algorithmic_flops_per_launch: {flops}", ""]
    return "\n".join(lines)


def read_traffic(path: str) -> Optional[int]:
    """The traffic figure of a summary, or None when it is missing or the kernel
    sources changed since it was taken."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`")):
            k, _, v = line.partition(":")
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_sha():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--algorithmic", type=int, required=True)
    t.add_argument("--command", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("--kernel", required=True)
    m.add_argument("--flops", type=int, required=True)
    m.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.what == "stats":
        print(stats_markdown(a.csv, a.command), end="")
    elif a.what == "mfma":
        print(mfma_markdown(a.csv, a.kernel, a.flops, a.command), end="")
    else:
        print(traffic_markdown(a.fetch_csv, a.write_csv, a.kernel, a.copy_mib, a.algorithmic, a.command), end="")


if __name__ == "__main__":
    main()
