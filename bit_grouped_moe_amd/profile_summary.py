"""Summaries of rocprofv3 runs of bench.py, written under profiles/.

    python -m bit_grouped_moe_amd.profile_summary trace DIR --cmd "..." --out FILE.md
    python -m bit_grouped_moe_amd.profile_summary traffic FETCH_DIR WRITE_DIR \
        --control-bytes B --cmd "..." --out FILE.md --json profiles/traffic_counters.json
    python -m bit_grouped_moe_amd.profile_summary counters DIR [DIR ...] --cmd "..." --out FILE.md \
        [--kernels all]

``trace`` reads the kernel trace (``*_kernel_trace.csv``) of a
``rocprofv3 --kernel-trace --stats --output-format csv`` run and tabulates
every libgq / probe kernel per launch shape (grid size in threads): calls,
median, mean, min and max device time.

``counters`` reads one or more ``rocprofv3 --pmc <SQ counters>`` runs of
``bench.py`` and tabulates, for the decode gate_up GEMV and the prefill
gate_up GEMM launches of the Qwen3 workload (or, with ``--kernels all``,
for every libgq kernel launch shape in the runs), the median per dispatch
of every counter collected, plus ratios formed from counters of the same
dispatch (no normalisation by unit counts or clocks).

``traffic`` reads two ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE``
runs of ``bench.py``.  The counters report KiB per dispatch; the factor that
turns them into bytes is taken from the plain copy control
(``gq_probe_copy``, ``--control-bytes`` read and written per launch), and
applied to the decode gate_up GEMV and the prefill gate_up GEMM launches of
the Qwen3 workload.  The JSON records the SHA-256 of the kernel sources, so
the bench reports traffic only while the sources are unchanged.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# Launch shapes (grid size in threads) of the bench's Qwen3 NF4 workloads.
GATE_UP_GEMV = ("grouped_gemv_kernel<false, 2, true, 0, false>", 393216)  # N=1536, K=2048, M=1, top-8
GATE_UP_GEMM = ("grouped_gemm_fwd_kernel<0>", 405504)      # M=4096 top-8, 257 x 6 tiles
SOURCES = {"gemv_nf4_gate_up_m1": ["gemv.hip", "gq_device.hpp"],
           "gemm_nf4_gate_up_prefill": ["gemm.hip", "gemm_common.hpp", "gq_device.hpp"]}


_PROBES = ("stream_read_kernel(", "copy_kernel(", "empty_kernel(")


def _short(name):
    """Kernel name with template arguments for libgq and probe kernels; None
    for any other kernel (torch's own)."""
    if name.startswith("gq::") or name.startswith("void gq::"):
        return name.split("gq::", 1)[1].split("(", 1)[0]
    if name.startswith("(anonymous namespace)::"):
        for key in _PROBES:
            if name.startswith("(anonymous namespace)::" + key):
                return key[:-1]
    return None


def sources_sha(key):
    h = hashlib.sha256()
    for f in SOURCES[key]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def trace(args):
    files = glob.glob(os.path.join(args.dir, "**", "*_kernel_trace.csv"), recursive=True)
    groups = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            k = _short(r["Kernel_Name"])
            if not k:
                continue
            grid = int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1)
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups.setdefault((k, grid, r["Workgroup_Size_X"]), []).append(us)
    lines = ["# rocprofv3 kernel trace: " + args.title, "",
             "Command (run from the repository root):", "", "```", args.cmd, "```", "",
             "| kernel | grid (threads) | block | calls | median us | mean us | min us | max us |",
             "|---|---|---|---|---|---|---|---|"]
    for (k, grid, wg), v in sorted(groups.items()):
        lines.append(f"| {k} | {grid} | {wg} | {len(v)} | {statistics.median(v):.2f} | "
                     f"{statistics.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    open(args.out, "w").write("\n".join(lines) + "\n")


def _counter(dirpath, name):
    out = {}
    for f in glob.glob(os.path.join(dirpath, "**", "*_counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != name:
                continue
            k = _short(r["Kernel_Name"])
            if not k:
                continue
            key = (k, int(r["Grid_Size"]), int(r["Dispatch_Id"]))
            out[key] = out.get(key, 0.0) + float(r["Counter_Value"])
    return out


def _median_for(values, kernel, grid=None):
    v = [x for (k, g, _), x in values.items()
         if k.startswith(kernel) and (grid is None or g == grid)]
    return statistics.median(v) if v else None


def traffic(args):
    fetch = _counter(args.fetch_dir, "FETCH_SIZE")
    write = _counter(args.write_dir, "WRITE_SIZE")
    grid = -(-args.control_bytes // (16 * 256)) * 256        # copy_kernel: 16 B/thread, 256/block
    cf = _median_for(fetch, "copy_kernel", grid)
    cw = _median_for(write, "copy_kernel", grid)
    if not cf or not cw:
        sys.exit("copy control not found in the counter runs")
    fr = args.control_bytes / (cf * 1024.0)
    fw = args.control_bytes / (cw * 1024.0)
    rec = {"factor_read": fr, "factor_write": fw, "control_bytes": args.control_bytes,
           "command": args.cmd}
    rows = []
    for key, (kern, grid) in (("gemv_nf4_gate_up_m1", GATE_UP_GEMV),
                              ("gemm_nf4_gate_up_prefill", GATE_UP_GEMM)):
        f = _median_for(fetch, kern, grid)
        w = _median_for(write, kern, grid)
        if f is None or w is None:
            continue
        fb, wb = f * 1024.0 * fr, w * 1024.0 * fw
        rec[key] = {"source": SOURCES[key][0], "source_sha256": sources_sha(key),
                    "fetch_bytes": fb, "write_bytes": wb, "hbm_bytes_per_launch": fb + wb}
        rows.append(f"| {key} | {kern} | {grid} | {f:.1f} | {w:.1f} | {fb:,.0f} | {wb:,.0f} |")
    if getattr(args, "kernels", "bench") == "all":
        rows.append("")
        rows.append("Every kernel launch shape in the runs (median per dispatch):")
        rows.append("")
        rows.append("| kernel | grid | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | written bytes |")
        rows.append("|---|---|---|---|---|---|")
        for kern, grid in sorted({(k, g) for (k, g, _) in fetch} & {(k, g) for (k, g, _) in write}):
            f = _median_for(fetch, kern, grid)
            w = _median_for(write, kern, grid)
            rows.append(f"| {kern} | {grid} | {f:.1f} | {w:.1f} | {f * 1024 * fr:,.0f} | "
                        f"{w * 1024 * fw:,.0f} |")
    json.dump(rec, open(args.json, "w"), indent=1)
    lines = ["# HBM traffic per launch from rocprofv3 counters: " + args.title, "",
             "Commands (run from the repository root):", "", "```", args.cmd, "```", "",
             f"Scale factors from the copy control ({args.control_bytes} bytes read and written "
             f"per launch): FETCH_SIZE x {fr:.4f}, WRITE_SIZE x {fw:.4f} "
             f"(raw KiB: fetch {cf:.1f}, write {cw:.1f}).", "",
             "| record | kernel | grid | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | written bytes |",
             "|---|---|---|---|---|---|---|"] + rows
    open(args.out, "w").write("\n".join(lines) + "\n")


_RATIOS = (
    ("VALU instructions per MFMA instruction", "SQ_INSTS_VALU", "SQ_INSTS_MFMA"),
    ("LDS instructions per MFMA instruction", "SQ_INSTS_LDS", "SQ_INSTS_MFMA"),
    ("LDS bank-conflict cycles per LDS instruction", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS"),
    ("cycles waves wait on LDS / wave cycles", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
    ("cycles waves wait on anything / wave cycles", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
    ("VALU+MFMA co-issue cycles / MFMA busy cycles", "SQ_VALU_MFMA_COEXEC_CYCLES",
     "SQ_VALU_MFMA_BUSY_CYCLES"),
    ("cycles waves wait on an instruction's data / wave cycles", "SQ_WAIT_INST_ANY",
     "SQ_WAVE_CYCLES"),
    # TA_TA_BUSY_sum adds the 256 per-CU address units, SQ_BUSY_CYCLES the 32
    # shader engines: (TA / 256) / (SQ / 32) is the busy fraction of one unit.
    ("address-unit busy fraction, (TA_TA_BUSY_sum / 256) / (SQ_BUSY_CYCLES / 32)",
     "TA_TA_BUSY_sum", "SQ_BUSY_CYCLES", 32 / 256),
    ("address unit stalled by the L1 / address-unit busy", "TA_ADDR_STALLED_BY_TC_CYCLES_sum",
     "TA_TA_BUSY_sum"),
)


def counters(args):
    every = getattr(args, "kernels", "bench") == "all"
    per = {}                                                 # (record, counter) -> [values]
    for d in args.dirs:
        for f in glob.glob(os.path.join(d, "**", "*_counter_collection.csv"), recursive=True):
            disp = {}
            for r in csv.DictReader(open(f)):
                k = _short(r["Kernel_Name"])
                if not k:
                    continue
                key = (k, int(r["Grid_Size"]), int(r["Dispatch_Id"]), r["Counter_Name"])
                disp[key] = disp.get(key, 0.0) + float(r["Counter_Value"])
            for (k, grid, _, cname), v in disp.items():
                if every:
                    per.setdefault((f"{k} grid {grid}", cname), []).append(v)
                    continue
                for rec, (kern, kgrid) in (("gemv_nf4_gate_up_m1", GATE_UP_GEMV),
                                           ("gemm_nf4_gate_up_prefill", GATE_UP_GEMM)):
                    if k.startswith(kern) and grid == kgrid:
                        per.setdefault((rec, cname), []).append(v)
    if every:
        recs = tuple(sorted({r for (r, _) in per}))
        match = [m for m in (getattr(args, "match", None) or "").split(",") if m]
        if match:
            recs = tuple(r for r in recs if any(r.startswith(m) for m in match))
        labels = dict(x.split("=", 1) for x in (getattr(args, "label", None) or []))
        per = {(labels.get(r, r), c): v for (r, c), v in per.items() if r in recs}
        recs = tuple(labels.get(r, r) for r in recs)
    else:
        recs = ("gemv_nf4_gate_up_m1", "gemm_nf4_gate_up_prefill")
    names = sorted({c for (_, c) in per})
    med = {key: statistics.median(v) for key, v in per.items()}
    lines = ["# SQ counters per launch from rocprofv3: " + args.title, "",
             "Commands (run from the repository root):", "", "```", args.cmd, "```", "",
             "Median over the launches of each kernel (counter values summed over the "
             "device for one dispatch).", "",
             "| counter | " + " | ".join(recs) + " |", "|---|" + "---|" * len(recs)]
    for c in names:
        lines.append(f"| {c} | " + " | ".join(
            f"{med[(r, c)]:,.0f}" if (r, c) in med else "-" for r in recs) + " |")
    lines += ["", "| ratio (same dispatch, medians) | " + " | ".join(recs) + " |",
              "|---|" + "---|" * len(recs)]
    for label, num, den, *scale in _RATIOS:
        vals = []
        for r in recs:
            a, b = med.get((r, num)), med.get((r, den))
            vals.append(f"{a / b * (scale[0] if scale else 1.0):.3f}" if a is not None and b else "-")
        lines.append(f"| {label} | " + " | ".join(vals) + " |")
    open(args.out, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--cmd", required=True)
    t.add_argument("--title", default="bench.py")
    t.add_argument("--out", required=True)
    c = sub.add_parser("traffic")
    c.add_argument("fetch_dir")
    c.add_argument("write_dir")
    c.add_argument("--control-bytes", type=int, required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--title", default="bench.py")
    c.add_argument("--out", required=True)
    c.add_argument("--json", required=True)
    c.add_argument("--kernels", default="bench", choices=("bench", "all"))
    k = sub.add_parser("counters")
    k.add_argument("dirs", nargs="+")
    k.add_argument("--cmd", required=True)
    k.add_argument("--title", default="bench.py")
    k.add_argument("--out", required=True)
    k.add_argument("--kernels", default="bench", choices=("bench", "all"))
    k.add_argument("--match", default=None,
                   help="with --kernels all: comma-separated kernel-name prefixes to keep")
    k.add_argument("--label", action="append",
                   help="with --kernels all: 'KERNEL grid G=column title' (repeatable)")
    args = ap.parse_args()
    {"trace": trace, "traffic": traffic, "counters": counters}[args.mode](args)


if __name__ == "__main__":
    main()
