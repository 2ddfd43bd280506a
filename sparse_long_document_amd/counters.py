"""Measurement helpers around rocprofv3 output (not part of the attention path).

  python -m sparse_long_document_amd.counters copy [--mib N]
      A plain elementwise copy (x * 1.0) of N MiB (default 512), run 5 times:
      the calibration kernel for the FETCH_SIZE / WRITE_SIZE counters, whose
      true traffic is known (N MiB read and N MiB written per dispatch).

  python -m sparse_long_document_amd.counters stats DIR --kernel NAME --command CMD --out FILE
      Markdown summary of a `rocprofv3 --kernel-trace --stats` output
      directory (per-kernel calls, average and total duration).

  python -m sparse_long_document_amd.counters traffic --workload W --fetch DIR --write DIR
          --copy-fetch DIR --copy-write DIR --out FILE [--mib N] [--kernel-hash H]
          [--md FILE --avg-us T --algorithmic-bytes A --commands FILE]
      HBM bytes per launch of the attention kernel from two `--pmc` runs,
      each counter scaled by (known bytes / counted bytes) of the copy
      kernel; merged into the JSON file FILE under key W.  With --md, also a
      markdown summary (T: measured average launch duration in us; A: the
      algorithmic bytes per launch; the commands listed from FILE).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

KERNEL_MATCH = "lf_attn_fwd"


def _csvs(d: str, suffix: str):
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def counter_per_dispatch(d: str, counter: str, match: str):
    """Median over dispatches of kernels whose name contains `match` of the
    counter's value summed over its instances (KiB per dispatch for the
    *_SIZE counters)."""
    per = {}
    for f in _csvs(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if match not in r["Kernel_Name"] or r["Counter_Name"] != counter:
                    continue
                key = (f, r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} values for kernels matching {match!r} under {d}")
    return statistics.median(per.values()), len(per)


def cmd_copy(args):
    import torch

    # one elementwise kernel, nothing else: reads N MiB, writes N MiB per
    # dispatch (the input's contents do not matter)
    n = (args.mib << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": args.mib, "dispatches": 5}))


def cmd_stats(args):
    rows = []
    for f in _csvs(args.dir, "kernel_stats.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {args.dir}")
    lines = [f"# rocprofv3 kernel statistics: {args.title}", "",
             "Command (from the repository root, after `cd /tmp && export TMPDIR=/tmp`):", "",
             "```", args.command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | total (ms) | share |",
             "|---|---|---|---|---|---|---|"]
    focus = None
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        short = name if len(name) <= 70 else name[:67] + "..."
        avg = float(r["AverageNs"]) / 1e3
        lines.append(f"| `{short}` | {r['Calls']} | {avg:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['Percentage']):.1f}% |")
        if args.kernel in name and focus is None:
            focus = avg
    if focus is not None:
        lines += ["", f"Average duration of `{args.kernel}`: **{focus:.2f} us** per launch."]
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(args):
    known_kib = float(args.mib << 10)
    cf, _ = counter_per_dispatch(args.copy_fetch, "FETCH_SIZE", args.copy_match)
    cw, _ = counter_per_dispatch(args.copy_write, "WRITE_SIZE", args.copy_match)
    # one launch may be several kernels (comma-separated): their per-dispatch
    # medians add up
    kf = kw = 0.0
    nf = nw = 0
    for name in args.kernel.split(","):
        f1, n1 = counter_per_dispatch(args.fetch, "FETCH_SIZE", name)
        w1, m1 = counter_per_dispatch(args.write, "WRITE_SIZE", name)
        kf, kw, nf, nw = kf + f1, kw + w1, max(nf, n1), max(nw, m1)
    ff, fw = known_kib / cf, known_kib / cw
    fetch_b, write_b = kf * ff * 1024.0, kw * fw * 1024.0
    if args.kernel_hash is None:
        from sparse_long_document_amd import backward_source_hash, kernel_source_hash

        args.kernel_hash = backward_source_hash() if args.kernel.startswith("lf_attn_bwd") else kernel_source_hash()
    ent = {"kernel_hash": args.kernel_hash,
           "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
           "dispatches_fetch": nf, "dispatches_write": nw,
           "copy_kib": known_kib, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_factor": ff, "write_factor": fw,
           "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
           "bytes_per_launch": fetch_b + write_b}
    data = {}
    if os.path.exists(args.out):
        with open(args.out) as fh:
            data = json.load(fh)
    data[args.workload] = ent
    with open(args.out, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({args.workload: ent}))
    if args.md:
        cmds = open(args.commands).read().strip() if args.commands else ""
        lines = [f"# HBM traffic of {args.kernel}: {args.workload}", "",
                 "Commands (from the repository root, after `cd /tmp && export TMPDIR=/tmp`), one counter per run:",
                 "", "```", cmds, "```", "",
                 f"Calibration: an elementwise copy of {args.mib} MiB ({known_kib:.0f} KiB read and written per "
                 f"dispatch) counts FETCH_SIZE = {cf:.0f} KiB and WRITE_SIZE = {cw:.0f} KiB per dispatch, so the "
                 f"factors are {ff:.4f} (fetch) and {fw:.4f} (write).", "",
                 f"| | counter (KiB / dispatch, median of {nf}) | x factor | bytes per launch |",
                 "|---|---|---|---|",
                 f"| fetch | {kf:.1f} | {ff:.4f} | {fetch_b / 1e6:.2f} MB |",
                 f"| write | {kw:.1f} | {fw:.4f} | {write_b / 1e6:.2f} MB |",
                 f"| total | | | **{(fetch_b + write_b) / 1e6:.2f} MB** |", ""]
        if args.algorithmic_bytes:
            a = float(args.algorithmic_bytes)
            lines += [f"Algorithmic bytes per launch ({args.alg_desc}): {a / 1e6:.2f} MB.  "
                      f"Counted / algorithmic = {(fetch_b + write_b) / a:.3f}.", ""]
        if args.avg_us:
            t = float(args.avg_us) * 1e-6
            lines += [f"At the measured {args.avg_us} us per launch: {(fetch_b + write_b) / t / 1e9:.0f} GB/s "
                      f"counted ({(fetch_b + write_b) / t / 8e12 * 100:.1f} % of 8 TB/s).", ""]
        lines += [f"Kernel source hash {args.kernel_hash}."]
        with open(args.md, "w") as fh:
            fh.write("\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m sparse_long_document_amd.counters")
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=512)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--kernel", default=KERNEL_MATCH)
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--workload", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-match", default="")
    t.add_argument("--kernel-hash", default=None, help="default: the current kernel sources")
    t.add_argument("--mib", type=int, default=512)
    t.add_argument("--out", required=True)
    t.add_argument("--md", default=None)
    t.add_argument("--avg-us", default=None)
    t.add_argument("--algorithmic-bytes", default=None)
    t.add_argument("--commands", default=None)
    t.add_argument("--kernel", default=KERNEL_MATCH, help="kernel-name substring the counters are taken for")
    t.add_argument("--alg-desc", default="q, k, v read and out written per (token, head); k_g, v_g of the "
                   "batch row; q_g of the global rows; the mask")
    args = ap.parse_args(argv)
    {"copy": cmd_copy, "stats": cmd_stats, "traffic": cmd_traffic}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
