"""Summarise rocprofv3 CSV output into the short text files kept under profiles/.

    python profsum.py stats  <rocprof_dir> <out.md> --cmd "<command>"
    python profsum.py traffic <fetch_dir> <write_dir> <kernel_regex> \
        <copy_bytes> <workload> <out.json> --cmd "<command>"
    python profsum.py pmc <kernel_regex> <workload> <out.md> <pmc_dir>... --cmd "<command>"

`stats` lists every kernel of a --kernel-trace --stats run (calls, average
and median duration).  `traffic` turns two --pmc runs (FETCH_SIZE, then
WRITE_SIZE; KiB per dispatch) into HBM bytes per launch of the matching
kernel, each scaled by what the same counter reads for a device copy of
`copy_bytes` bytes (the __amd_rocclr_copyBuffer dispatch of the same run),
and records the source hash of the kernels it was measured on.

This module only reads profiler output; it needs neither a GPU nor the
HIP library.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "long_context_pool_amd", "csrc")


def source_sha() -> str:
    """Hash of the kernel sources and of the build script (its flags shape
    the kernels too)."""
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))]
    files.append(os.path.join(os.path.dirname(CSRC), "build.py"))
    for path in files:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _find(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return max(hits, key=os.path.getmtime)  # the newest run


def short_name(name: str) -> str:
    name = name.replace("misa::(anonymous namespace)::", "").replace("void ", "")
    name = re.sub(r"\(.*", "", name)
    return name.strip()


def stats(d: str, out: str, cmd: str) -> None:
    rows = list(csv.DictReader(open(_find(d, "kernel_trace.csv"))))
    per = {}
    for r in rows:
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        per.setdefault(short_name(r["Kernel_Name"]), []).append(dur)
    lines = ["# rocprofv3 kernel statistics", "", f"Command: `{cmd}`", "",
             f"Kernels measured on the source tree with hash `{source_sha()}`.", "",
             "| kernel | calls | average us | median us | min us |", "|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {len(v)} | {statistics.mean(v):.1f} | {statistics.median(v):.1f} | "
                     f"{min(v):.1f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _counter(d: str, counter: str):
    rows = list(csv.DictReader(open(_find(d, "counter_collection.csv"))))
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def traffic(fetch_dir: str, write_dir: str, regex: str, copy_bytes: int, workload: str, out: str,
            cmd: str) -> None:
    res = {"workload": workload, "kernel_regex": regex, "source_sha": source_sha(), "command": cmd,
           "copy_bytes": copy_bytes}
    total = 0.0
    for name, counter, d in (("fetch", "FETCH_SIZE", fetch_dir), ("write", "WRITE_SIZE", write_dir)):
        vals = _counter(d, counter)
        # The calibration copy is the largest copyBuffer dispatch of the run.
        copies = [v for k, vs in vals.items() if "copyBuffer" in k for v in vs]
        kerns = {short_name(k): vs for k, vs in vals.items() if re.search(regex, k)}
        if not copies or not kerns:
            raise RuntimeError(f"{counter}: missing copy ({len(copies)}) or kernel ({len(kerns)}) dispatches")
        copy = max(copies)
        # A copy of copy_bytes reads and writes copy_bytes: counter KiB -> bytes factor.
        factor = copy_bytes / (copy * 1024.0)
        # One launch of the timed call = one dispatch of each matching kernel.
        kib = sum(statistics.median(v) for v in kerns.values())
        per_launch = kib * 1024.0 * factor
        res[name] = {"kernels": {k: statistics.median(v) for k, v in kerns.items()},
                     "counter_kib_per_launch": kib, "copy_counter_kib": copy, "scale": factor,
                     "bytes_per_launch": per_launch}
        total += per_launch
    res["bytes_per_launch"] = total
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")


# Chip constants for the derived ratios (MI355X: 256 compute units of 4 SIMDs
# in 8 XCDs; GRBM_GUI_ACTIVE comes summed over the XCDs, so one XCD's busy
# cycles are a eighth of it).
CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8


def pmc(dirs: list, regex: str, workload: str, out: str, cmd: str) -> None:
    """Median per dispatch of every counter collected for the kernels that
    match ``regex`` (one or more --pmc runs of the same command), plus
    ratios over the kernel's cycles G = GRBM_GUI_ACTIVE / XCDs: MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (G x SIMDs), VALU issue = 4 SQ_INSTS_VALU /
    (G x SIMDs) (a wave64 vector instruction holds a 16-lane SIMD four
    cycles), waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES, and instructions per
    MFMA instruction."""
    vals = {}
    for d in dirs:
        for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
            if not re.search(regex, r["Kernel_Name"]):
                continue
            k = short_name(r["Kernel_Name"])
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise RuntimeError(f"no dispatch of {regex!r} in {dirs}")
    lines = ["# rocprofv3 counters", "", f"Workload: {workload}", "", f"Command: `{cmd}`", "",
             f"Kernels measured on the source tree with hash `{source_sha()}`. Values are medians "
             "per dispatch; one --pmc pass per group of counters.", ""]
    for k, cs in sorted(vals.items()):
        med = {c: statistics.median(v) for c, v in cs.items()}
        lines += [f"## `{k}`", "", "| counter | median per dispatch |", "|---|---|"]
        lines += [f"| {c} | {v:.6g} |" for c, v in sorted(med.items())]
        gui = med.get("GRBM_GUI_ACTIVE")
        gui = gui / XCD_NUM if gui else None
        der = []
        if gui:
            der.append(("kernel cycles per XCD (GRBM_GUI_ACTIVE / 8)", gui))
        if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            der.append(("MFMA busy (% of SIMD cycles)",
                        100 * med["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMD_NUM)))
        if gui and "SQ_INSTS_VALU" in med:
            der.append(("VALU issue (% of SIMD cycles)", 100 * 4 * med["SQ_INSTS_VALU"] / (gui * SIMD_NUM)))
        if gui and "SQ_VALU_MFMA_COEXEC_CYCLES" in med:
            der.append(("VALU and MFMA together (% of SIMD cycles)",
                        100 * med["SQ_VALU_MFMA_COEXEC_CYCLES"] / (gui * SIMD_NUM)))
        if "SQ_WAIT_ANY" in med and med.get("SQ_WAVE_CYCLES"):
            der.append(("waves waiting (% of wave cycles)", 100 * med["SQ_WAIT_ANY"] / med["SQ_WAVE_CYCLES"]))
        # Memory pipeline, per compute unit (one TA, TD and TCP each):
        # busy or stalled cycles over the kernel's cycles.
        for c, name in (("TA_TA_BUSY", "TA (address unit) busy"),
                        ("TD_TD_BUSY", "TD (data unit) busy"),
                        ("TA_ADDR_STALLED_BY_TC_CYCLES", "TA stalled by the L1 cache"),
                        ("TCP_PENDING_STALL_CYCLES", "L1 cache stalled on data pending from L2")):
            if gui and c in med:
                der.append((f"{name} (% of CU cycles)", 100 * med[c] / (gui * CU_NUM)))
        if med.get("TCP_TCC_READ_REQ"):
            if "TCP_TCC_READ_REQ_LATENCY" in med:
                der.append(("L1-to-L2 read latency (cycles per request)",
                            med["TCP_TCC_READ_REQ_LATENCY"] / med["TCP_TCC_READ_REQ"]))
        if "SQ_INSTS_MFMA" in med and med["SQ_INSTS_MFMA"] > 0:
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM"):
                if c in med:
                    der.append((f"{c} per SQ_INSTS_MFMA", med[c] / med["SQ_INSTS_MFMA"]))
        if der:
            lines += ["", "| derived | value |", "|---|---|"]
            lines += [f"| {n} | {v:.3g} |" for n, v in der]
        lines.append("")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("out")
    a.add_argument("--cmd", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("regex")
    b.add_argument("copy_bytes", type=int)
    b.add_argument("workload")
    b.add_argument("out")
    b.add_argument("--cmd", required=True)
    c = sub.add_parser("pmc")
    c.add_argument("regex")
    c.add_argument("workload")
    c.add_argument("out")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--cmd", required=True)
    args = ap.parse_args()
    if args.cmd_name == "pmc":
        pmc(args.dirs, args.regex, args.workload, args.out, args.cmd)
    elif args.cmd_name == "stats":
        stats(args.dir, args.out, args.cmd)
    else:
        traffic(args.fetch_dir, args.write_dir, args.regex, args.copy_bytes, args.workload, args.out,
                args.cmd)


if __name__ == "__main__":
    main()
