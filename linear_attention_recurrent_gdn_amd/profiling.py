"""Summaries of rocprofv3 output for the committed profiles.

    python -m linear_attention_recurrent_gdn_amd.profiling trace <kernel_stats.csv> <out.md> "<command>"
    python -m linear_attention_recurrent_gdn_amd.profiling traffic <fetch_dir> <write_dir> \
        <out.md> "<command>" <kernel-substring> [copy_bytes]

`trace` keeps the per-kernel call count and average / min / max duration.
`traffic` turns two --pmc passes (FETCH_SIZE, then WRITE_SIZE, KiB per
dispatch) into HBM bytes per dispatch of the named kernel, each counter
scaled by what it reads for a plain device copy of known size in the same
run (the bench's bandwidth probe copies 4 GiB), and records a hash of the
kernel sources so a later reader can tell whether the numbers still apply.
The machine-readable figures sit in a ```json block of the markdown.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
DECODE_SOURCES = ("csrc/decode.hip", "csrc/gdn_device.hpp")
PREFILL_SOURCES = ("csrc/prefill.hip", "csrc/gdn_device.hpp")


def source_hash(rel_paths) -> str:
    h = hashlib.sha256()
    for rel in rel_paths:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_profile_block(md_path):
    """The ```json block of a committed profile summary, or None."""
    try:
        text = open(md_path).read()
    except OSError:
        return None
    if "```json" not in text:
        return None
    body = text.split("```json", 1)[1].split("```", 1)[0]
    return json.loads(body)


def _short(name, n=110):
    return name if len(name) <= n else name[: n - 3] + "..."


def trace_summary(stats_csv, out_md, command):
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# Kernel trace: {os.path.basename(out_md)[:-3]}", "", "Command:", "",
             f"    {command}", "", "| kernel | calls | avg us | min us | max us | % |",
             "|---|---|---|---|---|---|"]
    for r in rows[:20]:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f} | "
                     f"{float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    data = {r["Name"]: {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3}
            for r in rows[:20]}
    lines += ["", "```json", json.dumps(data, indent=1), "```", ""]
    open(out_md, "w").write("\n".join(lines))


def _counter_rows(d):
    path = glob.glob(os.path.join(d, "*counter_collection.csv"))[0]
    return list(csv.DictReader(open(path)))


def traffic_summary(fetch_dir, write_dir, out_md, command, kernel_sub, copy_bytes=4 << 30,
                    sources=DECODE_SOURCES):
    fetch, write = _counter_rows(fetch_dir), _counter_rows(write_dir)
    copy_kib = copy_bytes / 1024

    def copies(rows):
        return [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]

    cw = [x for x in copies(write) if abs(x - copy_kib) < 0.01 * copy_kib]
    if not cw:
        raise SystemExit("no copy dispatch of the calibration size in the WRITE_SIZE pass")
    # the FETCH_SIZE pass sees the same copies, in the same order
    cf_all = copies(fetch)
    cw_all = copies(write)
    cf = [f for f, w in zip(cf_all, cw_all) if abs(w - copy_kib) < 0.01 * copy_kib]
    f_scale = copy_kib / statistics.median(cf)
    w_scale = copy_kib / statistics.median(cw)
    kf = [float(r["Counter_Value"]) for r in fetch if kernel_sub in r["Kernel_Name"]]
    kw = [float(r["Counter_Value"]) for r in write if kernel_sub in r["Kernel_Name"]]
    kname = next(r["Kernel_Name"] for r in fetch if kernel_sub in r["Kernel_Name"])
    rd = statistics.mean(kf) * f_scale * 1024
    wr = statistics.mean(kw) * w_scale * 1024
    data = dict(kernel=kname, dispatches=len(kf), fetch_kib_raw=statistics.mean(kf),
                write_kib_raw=statistics.mean(kw), fetch_scale=f_scale, write_scale=w_scale,
                read_bytes=rd, write_bytes=wr, traffic_bytes=rd + wr,
                calibration=f"plain device copy of {copy_bytes} bytes: FETCH_SIZE "
                            f"{statistics.median(cf):.0f} KiB, WRITE_SIZE "
                            f"{statistics.median(cw):.0f} KiB per dispatch",
                source_hash=source_hash(sources))
    lines = [f"# HBM traffic: {os.path.basename(out_md)[:-3]}", "",
             "Two counter passes over the same command (FETCH_SIZE, then WRITE_SIZE):", "",
             f"    {command}", "",
             f"Kernel: `{_short(kname, 200)}` ({len(kf)} dispatches averaged).", "",
             f"- FETCH_SIZE {data['fetch_kib_raw']:.0f} KiB/dispatch x {f_scale:.4f} = "
             f"{rd/1e6:.1f} MB read",
             f"- WRITE_SIZE {data['write_kib_raw']:.0f} KiB/dispatch x {w_scale:.4f} = "
             f"{wr/1e6:.1f} MB written",
             f"- traffic {(rd+wr)/1e6:.1f} MB per dispatch",
             f"- scale factors from a {data['calibration']}", "",
             "```json", json.dumps(data, indent=1), "```", ""]
    open(out_md, "w").write("\n".join(lines))


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "trace":
        trace_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif mode == "traffic":
        extra = {}
        if len(sys.argv) > 7:
            extra["copy_bytes"] = int(sys.argv[7])
        traffic_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6], **extra)
    else:
        raise SystemExit(__doc__)
