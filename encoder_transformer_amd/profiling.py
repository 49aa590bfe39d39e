"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m encoder_transformer_amd.profiling stats <kernel_stats.csv> <out.md> --command "<cmd>"
    python -m encoder_transformer_amd.profiling traffic <fetch_counter.csv> <write_counter.csv> <out.md>
        --kernel layer_kernel --copy-mib 256 --command "<cmd>"
    python -m encoder_transformer_amd.profiling call_traffic <fetch.csv> <write.csv> <out.md> --calls N
        --copy-mib 256 --command "<cmd>"
    python -m encoder_transformer_amd.profiling counters <counter.csv> <out.md> --kernels a,b --title T
        --command "<cmd>"

`stats` turns rocprofv3's --stats kernel table into markdown.  `traffic`
turns two --pmc passes (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) into
HBM bytes per launch of one kernel: each counter is scaled by what it reads
for a plain device copy of known size in the same run (bench.py
--calibration-copy-mib), because FETCH_SIZE and WRITE_SIZE do not count
bytes one-to-one on every chip.  The summary carries a digest of the kernel
sources; bench.py reports the figure only while the digest still matches.
`call_traffic` does the same for every dispatch of a run of whole calls
(bench.py --latency-only) and reports HBM bytes per call.  `counters`
tabulates any --pmc pass per kernel (mean per dispatch) and, where the pass
holds SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE, the matrix-core
utilization as rocprofv3 defines it (MfmaUtil: the busy cycles summed over
the SIMDs, over one XCD's GUI-active cycles times the SIMD count).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# kernel class (as bench.py names it) -> device function and the sources it is built from
KERNELS = {
    "layer": ("layer_kernel", ["jl_layer.hip", "jl_rowblock.h", "jl_device.h", "jl_internal.h"]),
    "head_layer": ("head_kernel", ["jl_head.hip", "jl_rowblock.h", "jl_device.h", "jl_internal.h"]),
    "embed": ("embed_qkv_kernel", ["jl_embed.hip", "jl_rowblock.h", "jl_device.h", "jl_internal.h"]),
    "attn_global": ("attn_kernel", ["jl_kernels.hip", "jl_device.h", "jl_internal.h"]),
    "attn_local": ("attn_kernel", ["jl_kernels.hip", "jl_device.h", "jl_internal.h"]),
}
COPY_KERNEL = "copyBuffer"
# sources of the per-GEMM schedule that a batch-1 call runs (kernels and launch plan)
CALL_SOURCES = ["jl_kernels.hip", "jl_device.h", "jl_internal.h", "jl_api.cpp"]
CALL_TRAFFIC_LINE = re.compile(r"^traffic_bytes_per_call:\s*([0-9.]+)\s+sources_sha256:\s*([0-9a-f]+)\s*$", re.M)
SIMD_NUM = 1024  # 256 CUs x 4 SIMDs
TRAFFIC_LINE = re.compile(r"^traffic_bytes_per_launch:\s*([0-9.]+)\s+sources_sha256:\s*([0-9a-f]+)\s*$", re.M)


def source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def traffic_path(profiles_dir: str, cls: str) -> str:
    return os.path.join(profiles_dir, f"traffic_{KERNELS[cls][0]}_16x1024.md")


def read_traffic(profiles_dir: str, cls: str):
    """HBM bytes per launch of class `cls` from its committed summary, or None
    when there is none or the kernel sources changed since it was taken."""
    if cls not in KERNELS:
        return None
    path = traffic_path(profiles_dir, cls)
    if not os.path.exists(path):
        return None
    m = TRAFFIC_LINE.search(open(path).read())
    if not m or m.group(2) != source_digest(KERNELS[cls][1]):
        return None
    return float(m.group(1))


def _per_dispatch(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter of a --pmc CSV."""
    out = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def _select(table, name_part, min_grid=0):
    vals = [v for k, rows in table.items() if name_part in k for g, v in rows if g >= min_grid]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel named like {name_part!r}")
    return vals


def cmd_traffic(a):
    fetch = _per_dispatch(a.fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(a.write_csv, "WRITE_SIZE")
    copy_bytes = a.copy_mib * (1 << 20)
    # the calibration copy is the largest copy dispatch of the run
    cf = max(_select(fetch, COPY_KERNEL)) * 1024.0
    cw = max(_select(write, COPY_KERNEL)) * 1024.0
    f_scale, w_scale = copy_bytes / cf, copy_bytes / cw
    kf = _select(fetch, a.kernel)
    kw = _select(write, a.kernel)
    fb = statistics.mean(kf) * 1024.0 * f_scale
    wb = statistics.mean(kw) * 1024.0 * w_scale
    cls = next(c for c, (k, _) in KERNELS.items() if k == a.kernel)
    digest = source_digest(KERNELS[cls][1])
    lines = [
        f"# HBM traffic of `{a.kernel}` (16 x 1,024 tokens, bf16)",
        "",
        "Command (two passes, one counter each, from the repository root):",
        "",
        "```",
        a.command,
        "```",
        "",
        f"Calibration: a plain device copy of {a.copy_mib} MiB in the same run reads "
        f"FETCH_SIZE = {cf / 1024:.0f} KiB and WRITE_SIZE = {cw / 1024:.0f} KiB per dispatch, "
        f"so the counters are scaled by {f_scale:.3f} (fetch) and {w_scale:.3f} (write).",
        "",
        "| counter | dispatches | mean KiB per dispatch | scaled MB per launch |",
        "|---|---|---|---|",
        f"| FETCH_SIZE | {len(kf)} | {statistics.mean(kf):.1f} | {fb / 1e6:.2f} |",
        f"| WRITE_SIZE | {len(kw)} | {statistics.mean(kw):.1f} | {wb / 1e6:.2f} |",
        f"| total | | | {(fb + wb) / 1e6:.2f} |",
        "",
        f"traffic_bytes_per_launch: {fb + wb:.0f} sources_sha256: {digest}",
        "",
    ]
    if a.note:
        lines += [a.note, ""]
    with open(a.out_md, "w") as fh:
        fh.write("\n".join(lines))
    print(f"{a.out_md}: {(fb + wb) / 1e6:.2f} MB per launch")


def read_call_traffic(profiles_dir: str):
    """HBM bytes per 1 x 1,024 call from its committed summary, or None when
    there is none or the sources changed since it was taken."""
    path = os.path.join(profiles_dir, "traffic_call_1x1024_bf16.md")
    if not os.path.exists(path):
        return None
    m = CALL_TRAFFIC_LINE.search(open(path).read())
    if not m or m.group(2) != source_digest(CALL_SOURCES):
        return None
    return float(m.group(1))


def cmd_call_traffic(a):
    out = {}
    for c, path in (("FETCH_SIZE", a.fetch_csv), ("WRITE_SIZE", a.write_csv)):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == c]
        copies = [float(r["Counter_Value"]) for r in rows if COPY_KERNEL in r["Kernel_Name"]]
        cal = max(copies)  # the calibration copy: the largest copy dispatch
        scale = a.copy_mib * (1 << 20) / (cal * 1024.0)
        # every dispatch of the calls: all but the calibration copies
        total = sum(float(r["Counter_Value"]) for r in rows
                    if not (COPY_KERNEL in r["Kernel_Name"] and float(r["Counter_Value"]) > 0.5 * cal))
        out[c] = (len(rows), cal, scale, total * 1024.0 * scale / a.calls)
    fb, wb = out["FETCH_SIZE"][3], out["WRITE_SIZE"][3]
    digest = source_digest(CALL_SOURCES)
    lines = [
        "# HBM traffic of one 1 x 1,024 call (bf16, jl_forward + jl_probs)",
        "",
        "Command (two passes, one counter each, from the repository root):",
        "",
        "```",
        a.command,
        "```",
        "",
        f"Every dispatch of the {a.calls} calls of the run is summed (the three calibration copies of "
        f"{a.copy_mib} MiB excluded) and divided by {a.calls}.  Calibration: the copy reads "
        f"FETCH_SIZE = {out['FETCH_SIZE'][1]:.0f} KiB and WRITE_SIZE = {out['WRITE_SIZE'][1]:.0f} KiB per dispatch, "
        f"so the counters are scaled by {out['FETCH_SIZE'][2]:.3f} (fetch) and {out['WRITE_SIZE'][2]:.3f} (write).",
        "",
        "| counter | dispatches in the run | scaled MB per call |",
        "|---|---|---|",
        f"| FETCH_SIZE | {out['FETCH_SIZE'][0]} | {fb / 1e6:.2f} |",
        f"| WRITE_SIZE | {out['WRITE_SIZE'][0]} | {wb / 1e6:.2f} |",
        f"| total | | {(fb + wb) / 1e6:.2f} |",
        "",
        f"traffic_bytes_per_call: {fb + wb:.0f} sources_sha256: {digest}",
        "",
    ]
    if a.note:
        lines += [a.note, ""]
    with open(a.out_md, "w") as fh:
        fh.write("\n".join(lines))
    print(f"{a.out_md}: {(fb + wb) / 1e6:.2f} MB per call")


def gpu_xcc(counter_csv: str) -> int:
    """XCD count of the GPU agent, from the run_agent_info.csv beside a counter CSV."""
    info = os.path.join(os.path.dirname(counter_csv), "run_agent_info.csv")
    for r in csv.DictReader(open(info)):
        if r.get("Agent_Type", "").upper() == "GPU" or int(r.get("Simd_Count", "0") or 0) > 0:
            return int(r["Num_Xcc"])
    raise SystemExit("no GPU agent in " + info)


def cmd_counters(a):
    rows = list(csv.DictReader(open(a.counter_csv)))
    xcc = gpu_xcc(a.counter_csv)
    names = sorted({r["Counter_Name"] for r in rows})
    lines = [f"# Counters: {a.title}", "", "Command (from the repository root):", "", "```", a.command, "```", "",
             "Mean per dispatch of each kernel (counters summed over the chip's units as rocprofv3 reports them; "
             f"GRBM_GUI_ACTIVE is summed over the {xcc} XCDs, so one XCD's active cycles are it / {xcc}).",
             ""]
    have_util = "SQ_VALU_MFMA_BUSY_CYCLES" in names and "GRBM_GUI_ACTIVE" in names
    head = ["kernel", "dispatches"] + names + (["MFMA util"] if have_util else [])
    lines += ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    for part in a.kernels.split(";"):
        sel = [r for r in rows if part in r["Kernel_Name"]]
        if not sel:
            continue
        per = {}
        for r in sel:
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        n = len(per[names[0]]) if names[0] in per else 0
        vals = [statistics.mean(per[c]) if c in per else float("nan") for c in names]
        cells = [f"`{part}`", str(n)] + [f"{v:.4g}" for v in vals]
        if have_util:
            util = statistics.mean(per["SQ_VALU_MFMA_BUSY_CYCLES"]) / (
                statistics.mean(per["GRBM_GUI_ACTIVE"]) / xcc * SIMD_NUM)
            cells.append(f"{100 * util:.1f}%")
        lines.append("| " + " | ".join(cells) + " |")
    lines.append("")
    if a.note:
        lines += [a.note, ""]
    with open(a.out_md, "w") as fh:
        fh.write("\n".join(lines))
    print(a.out_md)


def cmd_stats(a):
    rows = []
    with open(a.stats_csv) as fh:
        for r in csv.DictReader(fh):
            rows.append(r)
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [
        f"# Kernel time: {a.title}",
        "",
        "Command (from the repository root):",
        "",
        "```",
        a.command,
        "```",
        "",
        "| kernel | calls | total ms | avg us | min us | max us | share |",
        "|---|---|---|---|---|---|---|",
    ]
    for r in rows[: a.top]:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(
            f"| `{name}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
            f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
            f"{float(r['MaxNs']) / 1e3:.2f} | {100 * float(r['TotalDurationNs']) / total:.1f}% |")
    lines += ["", f"All kernels: {total / 1e6:.3f} ms over {sum(int(r['Calls']) for r in rows)} dispatches.", ""]
    if a.note:
        lines += [a.note, ""]
    with open(a.out_md, "w") as fh:
        fh.write("\n".join(lines))
    print(a.out_md)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("out_md")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="16 x 1,024 tokens, bf16")
    s.add_argument("--top", type=int, default=25)
    s.add_argument("--note", default="")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("out_md")
    t.add_argument("--kernel", default="layer_kernel")
    t.add_argument("--copy-mib", type=int, default=256)
    t.add_argument("--command", required=True)
    t.add_argument("--note", default="")
    c = sub.add_parser("call_traffic")
    c.add_argument("fetch_csv")
    c.add_argument("write_csv")
    c.add_argument("out_md")
    c.add_argument("--calls", type=int, required=True)
    c.add_argument("--copy-mib", type=int, default=256)
    c.add_argument("--command", required=True)
    c.add_argument("--note", default="")
    k = sub.add_parser("counters")
    k.add_argument("counter_csv")
    k.add_argument("out_md")
    k.add_argument("--kernels", required=True, help="parts of kernel names, separated by ;")
    k.add_argument("--title", required=True)
    k.add_argument("--command", required=True)
    k.add_argument("--note", default="")
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "call_traffic": cmd_call_traffic, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
