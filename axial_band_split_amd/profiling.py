"""Summaries of rocprofv3 output for the measurement records under profiles/.

    python -m axial_band_split_amd.profiling stats    <kernel_stats.csv> <out.md> --command "<cmd>"
    python -m axial_band_split_amd.profiling counters <counter_collection.csv> <out.md> --command "<cmd>"
    python -m axial_band_split_amd.profiling traffic  <fetch.csv> <write.csv> <cal_fetch.csv> <cal_write.csv>
                                                      <kernel regex> <out.json> --command "<cmd>"
    python axial_band_split_amd/profiling.py calibrate   (run under rocprofv3 --pmc: one device copy)

`traffic` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of one kernel into bytes per launch,
each scaled by what the same counter reads for a plain device copy of known size (the calibration
runs), and records the hash of the kernel sources it was measured on, so a reader can tell when
the counters no longer describe the current code.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CAL_BYTES = 64 * 1024 * 1024 * 4      # the calibration copy moves 256 MiB in each direction


def short_name(k: str) -> str:
    k = k.replace("mbr::(anonymous namespace)::", "")
    m = re.match(r"_ZN3mbr12_GLOBAL__N_1(\d+)(\w+?)I(.*)E(E|Ev).*", k)
    if m:
        n = int(m.group(1))
        name = (m.group(2) + m.group(3))[:n] if len(m.group(2)) >= n else m.group(2)[:n]
        rest = k[len("_ZN3mbr12_GLOBAL__N_1") + len(m.group(1)) + n:]
        tparts = []
        if rest.startswith("IDF16_"):
            tparts.append("f16")
        elif rest.startswith("IDF16b"):
            tparts.append("bf16")
        elif rest.startswith("If"):
            tparts.append("f32")
        epi = re.search(r"Li(\d+)E", rest)
        if epi and name.startswith("gemm"):
            tparts.append(["embed", "qkv", "gelu", "resid", "tanh", "glu", "store16", "ffn2"][int(epi.group(1))])
        cfg = re.search(r"CfgILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", rest)
        if cfg:
            bm, wm, wn, ns = map(int, cfg.groups())
            tparts.append(f"{bm}x{64 * wn}/{wm}x{wn}w/{ns}st")
        blk = re.search(r"BlockCfgI\w+?Li(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", rest)
        if blk and name.startswith("block"):
            tparts.append(f"D{blk.group(1)}/I{blk.group(2)}/{blk.group(3)}st")
        dh = re.search(r"Li(\d+)EEEv", rest)
        if dh and name.startswith("attn"):
            tparts.append(f"dh{dh.group(1)}")
        return f"{name}<{','.join(tparts)}>"
    return k[:80]


def kernel_stats(csv_path: str) -> list:
    rows = list(csv.DictReader(open(csv_path)))
    out = []
    for r in rows:
        out.append(dict(name=short_name(r["Name"]), calls=int(r["Calls"]), total_ns=float(r["TotalDurationNs"]),
                        avg_ns=float(r["AverageNs"]), pct=float(r["Percentage"]), min_ns=float(r["MinNs"]),
                        max_ns=float(r["MaxNs"])))
    return out


def stats_md(csv_path: str, command: str) -> str:
    rows = kernel_stats(csv_path)
    lines = ["# rocprofv3 kernel statistics", "", f"Command: `{command}`", "",
             "| kernel | calls | avg us | min us | max us | total ms | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['name']} | {r['calls']} | {r['avg_ns'] / 1e3:.1f} | {r['min_ns'] / 1e3:.1f} | "
                     f"{r['max_ns'] / 1e3:.1f} | {r['total_ns'] / 1e6:.3f} | {r['pct']:.2f} |")
    return "\n".join(lines) + "\n"


def counter_means(csv_path: str, kernel_regex: str | None = None) -> dict:
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        if kernel_regex and not re.search(kernel_regex, r["Kernel_Name"]):
            continue
        agg[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in d.items()} | {"_dispatches": max(len(v) for v in d.values())}
            for k, d in agg.items()}


def counters_md(csv_path: str, command: str) -> str:
    means = counter_means(csv_path)
    names = sorted({c for d in means.values() for c in d if not c.startswith("_")})
    lines = ["# rocprofv3 counters (mean per dispatch)", "", f"Command: `{command}`", "",
             "| kernel | dispatches | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    for k, d in means.items():
        lines.append(f"| {k} | {d['_dispatches']} | " + " | ".join(f"{d.get(c, float('nan')):.4g}" for c in names) + " |")
    return "\n".join(lines) + "\n"


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _one(csv_path: str, counter: str, regex: str) -> float:
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if r["Counter_Name"] == counter and re.search(regex, r["Kernel_Name"])]
    if not vals:
        raise SystemExit(f"no {counter} rows for /{regex}/ in {csv_path}")
    return sum(vals) / len(vals)


def traffic_record(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, regex, command) -> dict:
    copy = r"copyBuffer|elementwise_kernel.*(copy|Copy)|direct_copy"
    fetch_kib = _one(fetch_csv, "FETCH_SIZE", regex)
    write_kib = _one(write_csv, "WRITE_SIZE", regex)
    cal_fetch = max(float(r["Counter_Value"]) for r in csv.DictReader(open(cal_fetch_csv))
                    if r["Counter_Name"] == "FETCH_SIZE" and re.search(copy, r["Kernel_Name"]))
    cal_write = max(float(r["Counter_Value"]) for r in csv.DictReader(open(cal_write_csv))
                    if r["Counter_Name"] == "WRITE_SIZE" and re.search(copy, r["Kernel_Name"]))
    ff, wf = CAL_BYTES / (cal_fetch * 1024), CAL_BYTES / (cal_write * 1024)
    return {"kernel_regex": regex, "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
            "fetch_factor": ff, "write_factor": wf,
            "bytes_per_launch": fetch_kib * 1024 * ff + write_kib * 1024 * wf,
            "calibration": f"device copy of {CAL_BYTES} bytes: FETCH_SIZE {cal_fetch:.0f} KiB, WRITE_SIZE {cal_write:.0f} KiB",
            "source_sha": source_hash(), "command": command}


def calibrate() -> None:
    """One device-to-device copy of CAL_BYTES on the GPU: the known-size kernel whose FETCH_SIZE and
    WRITE_SIZE readings scale the counters of the library's kernels."""
    import torch
    x = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    print(f"copied {CAL_BYTES} bytes", flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats"); a.add_argument("csv"); a.add_argument("out"); a.add_argument("--command", required=True)
    b = sub.add_parser("counters"); b.add_argument("csv"); b.add_argument("out"); b.add_argument("--command", required=True)
    c = sub.add_parser("traffic")
    for n in ("fetch", "write", "cal_fetch", "cal_write", "regex", "out"):
        c.add_argument(n)
    c.add_argument("--command", required=True)
    sub.add_parser("calibrate")
    args = ap.parse_args(argv)
    if args.what == "calibrate":
        calibrate()
        return 0
    if args.what == "stats":
        open(args.out, "w").write(stats_md(args.csv, args.command))
    elif args.what == "counters":
        open(args.out, "w").write(counters_md(args.csv, args.command))
    else:
        rec = traffic_record(args.fetch, args.write, args.cal_fetch, args.cal_write, args.regex, args.command)
        json.dump(rec, open(args.out, "w"), indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
