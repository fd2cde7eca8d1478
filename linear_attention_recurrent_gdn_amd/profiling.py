"""Summaries of rocprofv3 output for the committed profiles.

    python -m linear_attention_recurrent_gdn_amd.profiling trace <kernel_trace.csv> <out.md> "<command>"
    python -m linear_attention_recurrent_gdn_amd.profiling counters <out.md> "<command>" \
        <kernel-substring> <pass_dir> [<pass_dir> ...] [--sources attention|decode|prefill] \
        [--grid N]
    python -m linear_attention_recurrent_gdn_amd.profiling traffic <fetch_dir> <write_dir> \
        <out.md> "<command>" <kernel-substring> [--grid N] [--copy-bytes B] [--per-call K] \
        [--sources decode|prefill]

`counters` averages every counter of one or more --pmc passes per dispatch
of the named kernel (e.g. SQ_* utilisation and LDS counters).
`trace` keeps, per kernel and launch grid, the call count and the average /
min / max duration (one kernel serves workloads of different sizes, told
apart by their grids). `traffic` turns two --pmc passes (FETCH_SIZE, then
WRITE_SIZE, KiB per dispatch) into HBM bytes per dispatch of the named
kernel (optionally only its dispatches of one grid size), each counter
scaled by what it reads for a plain device copy of known size in the same
run (the bench's bandwidth probe copies 4 GiB), and records a hash of the
kernel sources so a later reader can tell whether the numbers still apply.
--per-call K records that one call of the operation launches the kernel K
times at that grid (a prefill in K segments), so per-call bytes are K times
the per-dispatch mean.
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
DECODE_SOURCES = ("csrc/decode_kernels.hpp", "csrc/decode_d128.hip", "csrc/gdn_device.hpp")
PREFILL_SOURCES = ("csrc/prefill_kernels.hpp", "csrc/prefill_d128.hip", "csrc/gdn_device.hpp")
ATTENTION_SOURCES = ("csrc/attention.hip", "csrc/attention_launch.hpp", "csrc/gdn_device.hpp")
SOURCES = {"decode": DECODE_SOURCES, "prefill": PREFILL_SOURCES, "attention": ATTENTION_SOURCES}


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


def trace_summary(trace_csv, out_md, command, top=24):
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in groups.values()) or 1.0
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:top]
    lines = [f"# Kernel trace: {os.path.basename(out_md)[:-3]}", "", "Command:", "",
             f"    {command}", "", "| kernel | grid | calls | avg us | min us | max us | % |",
             "|---|---|---|---|---|---|---|"]
    data = []
    for (name, grid), d in rows:
        avg = statistics.mean(d)
        lines.append(f"| `{_short(name)}` | {grid} | {len(d)} | {avg:.1f} | {min(d):.1f} | "
                     f"{max(d):.1f} | {100 * sum(d) / total:.1f} |")
        data.append({"kernel": name, "grid": grid, "calls": len(d), "avg_us": avg,
                     "median_us": statistics.median(d)})
    lines += ["", "```json", json.dumps(data, indent=1), "```", ""]
    open(out_md, "w").write("\n".join(lines))


def _counter_rows(d):
    path = glob.glob(os.path.join(d, "*counter_collection.csv"))[0]
    return list(csv.DictReader(open(path)))


def traffic_summary(fetch_dir, write_dir, out_md, command, kernel_sub, copy_bytes=4 << 30,
                    sources=DECODE_SOURCES, grid=None, per_call=1):
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
    def mine(r):
        return kernel_sub in r["Kernel_Name"] and (grid is None or int(r["Grid_Size"]) == grid)

    kf = [float(r["Counter_Value"]) for r in fetch if mine(r)]
    kw = [float(r["Counter_Value"]) for r in write if mine(r)]
    kname = next(r["Kernel_Name"] for r in fetch if mine(r))
    rd = statistics.mean(kf) * f_scale * 1024
    wr = statistics.mean(kw) * w_scale * 1024
    data = dict(kernel=kname, grid=grid, dispatches=len(kf), fetch_kib_raw=statistics.mean(kf),
                write_kib_raw=statistics.mean(kw), fetch_scale=f_scale, write_scale=w_scale,
                read_bytes=rd, write_bytes=wr, traffic_bytes=rd + wr, dispatches_per_call=per_call,
                calibration=f"plain device copy of {copy_bytes} bytes: FETCH_SIZE "
                            f"{statistics.median(cf):.0f} KiB, WRITE_SIZE "
                            f"{statistics.median(cw):.0f} KiB per dispatch",
                source_hash=source_hash(sources))
    lines = [f"# HBM traffic: {os.path.basename(out_md)[:-3]}", "",
             "Two counter passes over the same command (FETCH_SIZE, then WRITE_SIZE):", "",
             f"    {command}", "",
             f"Kernel: `{_short(kname, 200)}`"
             + (f", grid {grid}" if grid is not None else "")
             + f" ({len(kf)} dispatches averaged).", "",
             f"- FETCH_SIZE {data['fetch_kib_raw']:.0f} KiB/dispatch x {f_scale:.4f} = "
             f"{rd/1e6:.1f} MB read",
             f"- WRITE_SIZE {data['write_kib_raw']:.0f} KiB/dispatch x {w_scale:.4f} = "
             f"{wr/1e6:.1f} MB written",
             f"- traffic {(rd+wr)/1e6:.1f} MB per dispatch"
             + (f", {per_call} dispatches per call: {per_call*(rd+wr)/1e6:.1f} MB per call"
                if per_call > 1 else ""),
             f"- scale factors from a {data['calibration']}", "",
             "```json", json.dumps(data, indent=1), "```", ""]
    open(out_md, "w").write("\n".join(lines))


def counters_summary(out_md, command, kernel_sub, pass_dirs, sources=ATTENTION_SOURCES,
                     grid=None):
    vals, kname = {}, None
    for d in pass_dirs:
        for r in _counter_rows(d):
            if kernel_sub not in r["Kernel_Name"]:
                continue
            if grid is not None and int(r["Grid_Size"]) != grid:
                continue
            kname = kname or r["Kernel_Name"]
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no dispatch of {kernel_sub} in {pass_dirs}")
    data = {c: statistics.mean(v) for c, v in sorted(vals.items())}
    lines = [f"# Counters: {os.path.basename(out_md)[:-3]}", "",
             "Command (one --pmc pass per counter group):", "", f"    {command}", "",
             f"Kernel: `{_short(kname, 200)}`" + (f", grid {grid}" if grid is not None else "")
             + " (mean per dispatch).", "",
             "| counter | per dispatch |", "|---|---|"]
    lines += [f"| {c} | {v:.4g} |" for c, v in data.items()]
    block = dict(kernel=kname, grid=grid, counters=data, source_hash=source_hash(sources))
    lines += ["", "```json", json.dumps(block, indent=1), "```", ""]
    open(out_md, "w").write("\n".join(lines))


def main(argv):
    import argparse

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("trace_csv")
    t.add_argument("out_md")
    t.add_argument("command")
    f = sub.add_parser("traffic")
    for name in ("fetch_dir", "write_dir", "out_md", "command", "kernel_sub"):
        f.add_argument(name)
    f.add_argument("--grid", type=int, default=None)
    f.add_argument("--copy-bytes", type=int, default=4 << 30)
    f.add_argument("--per-call", type=int, default=1)
    f.add_argument("--sources", choices=("decode", "prefill"), default="decode")
    c = sub.add_parser("counters")
    c.add_argument("out_md")
    c.add_argument("command")
    c.add_argument("kernel_sub")
    c.add_argument("pass_dirs", nargs="+")
    c.add_argument("--sources", choices=tuple(SOURCES), default="attention")
    c.add_argument("--grid", type=int, default=None)
    a = ap.parse_args(argv)
    if a.mode == "trace":
        trace_summary(a.trace_csv, a.out_md, a.command)
    elif a.mode == "counters":
        counters_summary(a.out_md, a.command, a.kernel_sub, a.pass_dirs, SOURCES[a.sources],
                         grid=a.grid)
    else:
        traffic_summary(a.fetch_dir, a.write_dir, a.out_md, a.command, a.kernel_sub,
                        copy_bytes=a.copy_bytes, grid=a.grid, per_call=a.per_call,
                        sources=DECODE_SOURCES if a.sources == "decode" else PREFILL_SOURCES)


if __name__ == "__main__":
    main(sys.argv[1:])
