"""Condense rocprofv3 CSV output into the short text summaries kept under
``profiles/``.

Three commands:

* ``stats``: per-kernel duration table from ``*_kernel_trace.csv`` (all
  dispatches, and the last ``--last`` dispatches of ``--kernel``, which are the
  timed region when ``bench.py`` runs with no K sweep and no CPU baseline).
* ``traffic``: HBM bytes per dispatch of ``--kernel`` from two ``--pmc`` runs
  (``FETCH_SIZE`` and ``WRITE_SIZE``, KiB per dispatch).  Each counter is
  scaled by what it reads for the largest plain device-to-device copy in the
  same run (``bench.py --copy-probe-mib``), whose true size is known.
* ``mfma``: MFMA rate and busy fraction per kernel from one ``--pmc`` run of
  ``SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16
  SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE``: FLOPs = MOPS x 512 over the
  dispatch's own duration, against the dense bf16 / fp16 peak; busy % =
  MFMA busy cycles / (GPU active cycles per XCC x SIMDs).
* ``counters``: per-kernel means of whatever counters one ``--pmc`` run
  took, plus the ratios that explain where a kernel's waves spend their time
  when the run has the counters for them: VALU and MFMA instructions per
  wave, the share of wave cycles waiting on anything (``SQ_WAIT_ANY``) and
  waiting to issue (``SQ_WAIT_INST_ANY``), and MFMA busy %.

Usage::

    python -m greedy_block_verification_amd.rocprof_summary stats \\
        --trace DIR/q8b_kernel_trace.csv --kernel "sv::k_gemm_bf16<1, 2, 8, false>" --last 2160 \\
        --skip 720 --command "..." --out profiles/verify_q8b_k4_kernel_trace.md
    python -m greedy_block_verification_amd.rocprof_summary traffic \\
        --fetch A/q8b_counter_collection.csv --write B/q8b_counter_collection.csv \\
        --kernel "sv::k_gemm_bf16<1, 2, 8, false>" --last 1440 --skip 720 --copy-bytes 1073741824 \\
        --algorithmic-bytes 201659392 --command "..." --out profiles/gate_up_q8b_traffic.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(HERE, "csrc", "sv_kernels.hip")


def _short(name: str) -> str:
    return name.split("(")[0] if "(" in name else name


def _matches(name: str, kernel: str) -> bool:
    # "void sv::k_gemm_bf16<1, 2, 8, false>(sv::GemmArgs)" matches "sv::k_gemm_bf16<1, 2, 8, false>"
    n = name[5:] if name.startswith("void ") else name
    return n.startswith(kernel)


def kernel_source_sha256() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()


def stats(args):
    rows = list(csv.DictReader(open(args.trace)))
    per = defaultdict(list)
    for r in rows:
        per[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    total = sum(e - s for v in per.values() for s, e in v)
    lines = [f"# rocprofv3 kernel trace: {args.title}", "", "Command:", "", "```", args.command, "```", ""]
    sel = [v for k, v in per.items() if _matches(k, args.kernel)]
    if sel:
        d = sorted(sel[0], key=lambda t: t[0])
        d = d[len(d) - args.skip - args.last: len(d) - args.skip]
        durs = sorted((e - s) / 1000.0 for s, e in d)
        mean = sum(durs) / len(durs)
        tail = f" (before the final {args.skip})" if args.skip else ""
        lines += [f"Timed region: last {len(durs)} dispatches{tail} of `{args.kernel}`: mean {mean:.2f} us, "
                  f"median {durs[len(durs) // 2]:.2f} us, min {durs[0]:.2f} us, max {durs[-1]:.2f} us.", ""]
    lines += ["All dispatches of the run (warm-up, prefill and baseline decode included):", "",
              "| kernel | calls | mean us | total ms | share |", "|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(e - s for s, e in kv[1]))[:args.top]:
        t = sum(e - s for s, e in v)
        lines.append(f"| `{_short(k)}` | {len(v)} | {t / len(v) / 1000:.2f} | {t / 1e6:.2f} | {100 * t / total:.1f} % |")
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter(path, kernel, last, skip=0):
    rows = list(csv.DictReader(open(path)))
    copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
    vals = [(int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in rows if _matches(r["Kernel_Name"], kernel)]
    vals = [v for _, v in sorted(vals)]
    vals = vals[len(vals) - skip - last: len(vals) - skip]
    return max(copies), sum(vals) / len(vals), len(vals), rows[0]["Counter_Name"]


def traffic(args):
    cf, f_kib, nf, name_f = _counter(args.fetch, args.kernel, args.last, args.skip)
    cw, w_kib, nw, name_w = _counter(args.write, args.kernel, args.last, args.skip)
    assert name_f == "FETCH_SIZE" and name_w == "WRITE_SIZE", (name_f, name_w)
    scale_f = args.copy_bytes / (cf * 1024.0)
    scale_w = args.copy_bytes / (cw * 1024.0)
    fetch = f_kib * 1024.0 * scale_f
    write = w_kib * 1024.0 * scale_w
    rec = {
        "kernel": args.kernel,
        "kernel_source_sha256": kernel_source_sha256(),
        "dispatches": {"fetch": nf, "write": nw},
        "fetch_kib_per_dispatch": round(f_kib, 2), "write_kib_per_dispatch": round(w_kib, 2),
        "copy_probe_bytes": args.copy_bytes,
        "copy_probe_fetch_kib": cf, "copy_probe_write_kib": cw,
        "fetch_scale": round(scale_f, 4), "write_scale": round(scale_w, 4),
        "fetch_bytes_per_launch": int(fetch), "write_bytes_per_launch": int(write),
        "traffic_bytes_per_launch": int(fetch + write),
        "algorithmic_bytes_per_launch": args.algorithmic_bytes,
        "traffic_over_algorithmic": round((fetch + write) / args.algorithmic_bytes, 4) if args.algorithmic_bytes else None,
        "command": args.command,
    }
    json.dump(rec, open(args.out, "w"), indent=1)
    print(json.dumps(rec, indent=1))
    if args.table_out:
        _table(args, scale_f, scale_w)


def _per_kernel(path, last):
    per = defaultdict(list)
    for r in csv.DictReader(open(path)):
        per[r["Kernel_Name"]].append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return {k: [v for _, v in sorted(x)][-last:] for k, x in per.items()}


def _table(args, scale_f, scale_w):
    f, w = _per_kernel(args.fetch, args.table_last), _per_kernel(args.write, args.table_last)
    lines = [f"# HBM traffic per dispatch (scaled FETCH_SIZE / WRITE_SIZE): {args.title}", "",
             "Commands:", "", "```", args.command, "```", "",
             f"Scale factors from the largest plain device-to-device copy ({args.copy_bytes} bytes): "
             f"FETCH_SIZE x {scale_f:.4f}, WRITE_SIZE x {scale_w:.4f}.  Means over the last "
             f"{args.table_last} dispatches of each kernel.", "",
             "| kernel | fetch MB | write MB |", "|---|---|---|"]
    for k in sorted(f, key=lambda k: -sum(f[k]) / len(f[k])):
        if "copyBuffer" in k or k not in w:
            continue
        fm = sum(f[k]) / len(f[k]) * 1024 * scale_f / 1e6
        wm = sum(w[k]) / len(w[k]) * 1024 * scale_w / 1e6
        lines.append(f"| `{_short(k)}` | {fm:.3f} | {wm:.3f} |")
    open(args.table_out, "w").write("\n".join(lines) + "\n")


PEAK_MFMA_16BIT_TFLOPS = 2500.0   # dense bf16 / fp16


def mfma(args):
    per = defaultdict(lambda: defaultdict(dict))
    for r in csv.DictReader(open(args.counters)):
        d = per[r["Kernel_Name"]][int(r["Dispatch_Id"])]
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    need = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
    lines = [f"# MFMA rate per kernel: {args.title}", "", "Command:", "", "```", args.command, "```", "",
             f"FLOPs = (MOPS_BF16 + MOPS_F16) x 512 per dispatch over its duration; peak {PEAK_MFMA_16BIT_TFLOPS:.0f} "
             f"TFLOP/s dense 16-bit.  Busy % = MFMA busy cycles / (GRBM_GUI_ACTIVE / {args.xcc} XCCs x "
             f"{args.simds} SIMDs).  Means over the last {args.last} dispatches of each kernel.", "",
             "| kernel | dispatches | mean us | MFMA GFLOP per dispatch | MFMA TFLOP/s | % of peak | MFMA busy % |",
             "|---|---|---|---|---|---|---|"]
    rows = []
    for k, ds in per.items():
        ds = [ds[i] for i in sorted(ds)][-args.last:]
        ds = [d for d in ds if all(n in d for n in need)]
        if not ds:
            continue
        ns = sum(d["ns"] for d in ds) / len(ds)
        fl = sum((d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + d["SQ_INSTS_VALU_MFMA_MOPS_F16"]) * 512 for d in ds) / len(ds)
        if fl <= 0:
            continue
        busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds) / len(ds)
        gui = sum(d["GRBM_GUI_ACTIVE"] for d in ds) / len(ds)
        tf = fl / ns / 1e3
        util = 100.0 * busy / (gui / args.xcc * args.simds) if gui > 0 else 0.0
        rows.append((tf, f"| `{_short(k)}` | {len(ds)} | {ns / 1000:.2f} | {fl / 1e9:.2f} | {tf:.1f} | "
                         f"{100 * tf / PEAK_MFMA_16BIT_TFLOPS:.1f} | {util:.1f} |"))
    lines += [r for _, r in sorted(rows, key=lambda x: -x[0])]
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counters(args):
    per = defaultdict(lambda: defaultdict(dict))
    names = []
    for r in csv.DictReader(open(args.counters)):
        if args.kernel and not any(_matches(r["Kernel_Name"], k) for k in args.kernel):
            continue
        d = per[r["Kernel_Name"]][int(r["Dispatch_Id"])]
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if r["Counter_Name"] not in names:
            names.append(r["Counter_Name"])
    lines = [f"# Counters per kernel: {args.title}", "", "Command:", "", "```", args.command, "```", "",
             f"Means per dispatch over the last {args.last} dispatches of each kernel.", ""]
    derived = []
    if {"SQ_INSTS_VALU", "SQ_WAVES"} <= set(names):
        derived.append(("VALU / wave", lambda d: d["SQ_INSTS_VALU"] / d["SQ_WAVES"]))
    if {"SQ_INSTS_MFMA", "SQ_WAVES"} <= set(names):
        derived.append(("MFMA / wave", lambda d: d["SQ_INSTS_MFMA"] / d["SQ_WAVES"]))
    if {"SQ_WAIT_ANY", "SQ_WAVE_CYCLES"} <= set(names):
        derived.append(("wait any %", lambda d: 100.0 * d["SQ_WAIT_ANY"] / d["SQ_WAVE_CYCLES"]))
    if {"SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"} <= set(names):
        derived.append(("wait issue %", lambda d: 100.0 * d["SQ_WAIT_INST_ANY"] / d["SQ_WAVE_CYCLES"]))
    if {"SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"} <= set(names):
        derived.append(("MFMA busy %", lambda d: 100.0 * d["SQ_VALU_MFMA_BUSY_CYCLES"] /
                        (d["GRBM_GUI_ACTIVE"] / args.xcc * args.simds)))
    head = ["kernel", "dispatches", "mean us"] + names + [n for n, _ in derived]
    lines += ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    for k, ds in sorted(per.items(), key=lambda kv: kv[0]):
        ds = [ds[i] for i in sorted(ds)][-args.last:]
        ds = [d for d in ds if all(n in d for n in names)]
        if not ds:
            continue
        mean = {n: sum(d[n] for d in ds) / len(ds) for n in names + ["ns"]}
        cells = [f"`{_short(k)}`", str(len(ds)), f"{mean['ns'] / 1000:.2f}"]
        cells += [f"{mean[n]:.4g}" for n in names]
        for _, f in derived:
            try:
                cells.append(f"{f(mean):.3g}")
            except ZeroDivisionError:
                cells.append("-")
        lines.append("| " + " | ".join(cells) + " |")
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--trace", required=True)
    s.add_argument("--kernel", required=True)
    s.add_argument("--last", type=int, required=True)
    s.add_argument("--skip", type=int, default=0, help="dispatches after the timed region (bench.py's profiling pass)")
    s.add_argument("--top", type=int, default=16)
    s.add_argument("--title", default="")
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--last", type=int, required=True)
    t.add_argument("--skip", type=int, default=0)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--algorithmic-bytes", type=int, default=0)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--table-out", default="")
    t.add_argument("--table-last", type=int, default=200)
    t.add_argument("--title", default="")
    m = sub.add_parser("mfma")
    m.add_argument("--counters", required=True)
    m.add_argument("--last", type=int, default=1000)
    m.add_argument("--xcc", type=int, default=8)
    m.add_argument("--simds", type=int, default=1024)
    m.add_argument("--title", default="")
    m.add_argument("--command", required=True)
    m.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--counters", required=True)
    c.add_argument("--kernel", action="append", default=[], help="keep only kernels whose name starts so")
    c.add_argument("--last", type=int, default=1000)
    c.add_argument("--xcc", type=int, default=8)
    c.add_argument("--simds", type=int, default=1024)
    c.add_argument("--title", default="")
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    {"stats": stats, "traffic": traffic, "mfma": mfma, "counters": counters}[a.cmd](a)


if __name__ == "__main__":
    main()
