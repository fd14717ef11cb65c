"""Summaries of rocprofv3 output for the measurement records under profiles/.

    python -m axial_band_split_amd.profiling stats    <kernel_stats.csv> <out.md> --command "<cmd>"
    python -m axial_band_split_amd.profiling counters <counter_collection.csv> <out.md> --command "<cmd>"
    python -m axial_band_split_amd.profiling traffic  <fetch.csv> <write.csv> <cal_fetch.csv> <cal_write.csv>
                                                      <kernel regex> <out.json> --command "<cmd>"
    python axial_band_split_amd/profiling.py calibrate   (run under rocprofv3 --pmc: one device copy)
    python -m axial_band_split_amd.profiling sweep <bench line .json> ... <out.md> --command "<cmd>"
    python -m axial_band_split_amd.profiling roofline <kernel_stats.csv> <fetch.csv> <write.csv> <cal_fetch.csv>
                                                      <cal_write.csv> <sq.csv> <workload> <out.md> --command "<cmd>"
    python -m axial_band_split_amd.profiling waves <pass1.csv> <pass2.csv> <workload> <out.md> --command "<cmd>"

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
    # rocprofv3 prints gemm2_kernel<bf16, EPI_QKV, Cfg> (mangled ...gemm2_kernelIDF16bLi1E...) demangled
    # with its first two template arguments garbled; every other instantiation arrives mangled
    m = re.match(r"void gemm2_kernel<bool _Accum, int, E, Cfg<(\d+), (\d+), (\d+), (\d+)> >", k)
    if m:
        bm, wm, wn, ns = map(int, m.groups())
        return f"gemm2_kernel<bf16,qkv,{bm}x{64 * wn}/{wm}x{wn}w/{ns}st>"
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


# the sources a kernel class is built and launched from: a counter record stays valid while these
# are unchanged (changes to other kernels do not touch it)
KIND_SOURCES = {
    "block": ("k_block.hip", "kcommon.h", "kernels.h", "mbr_core.cpp"),
}


def source_hash(files=None) -> str:
    """Hash of the named files under csrc/ (all kernel sources when None)."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    names = sorted(files) if files else sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h", ".cpp")))
    for f in names:
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _one(csv_path: str, counter: str, regex: str) -> float:
    """Mean of a counter per dispatch for each kernel the pattern matches, summed over those kernels
    (a kernel class launched as several kernels, e.g. the fused block's two instantiations, counts
    as one launch of all of them)."""
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter and re.search(regex, r["Kernel_Name"]):
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    if not per:
        raise SystemExit(f"no {counter} rows for /{regex}/ in {csv_path}")
    return sum(sum(v) / len(v) for v in per.values())


def traffic_record(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, regex, command, sources=None) -> dict:
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
            "source_files": list(sources) if sources else None, "source_sha": source_hash(sources),
            "command": command}


N_SIMD, N_XCD = 1024, 8      # MI355X: 256 compute units x 4 SIMDs, 8 XCDs


def roofline_md(stats_csv, fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, sq_csv, workload, command) -> str:
    """Per kernel class of one forward: rocprofv3 average duration, algorithmic work against the
    MI355X peak, calibrated HBM bytes and the matrix-core busy fraction from the SQ counters."""
    import re as _re
    sys.path.insert(0, os.path.dirname(HERE))
    from axial_band_split_amd import roofline as R, synth, binding
    w = synth.WORKLOADS[workload]
    _, total_width, _ = binding.mbr_core_table_sizes(binding.config(w))
    shp = R.shape_of(w, total_width)
    flops = R.flops_per_launch(shp)
    flops["mask_hidden"] = (flops["mask_hidden_first"] + (w.mask_depth - 1) * flops["mask_hidden_next"]) / w.mask_depth
    byts = R.bytes_per_launch(shp)
    byts["norm"] = byts["norm_out"]
    stats = list(csv.DictReader(open(stats_csv)))
    cal_f = max(float(r["Counter_Value"]) for r in csv.DictReader(open(cal_fetch_csv)) if r["Counter_Name"] == "FETCH_SIZE")
    cal_w = max(float(r["Counter_Value"]) for r in csv.DictReader(open(cal_write_csv)) if r["Counter_Name"] == "WRITE_SIZE")
    ff, wf = CAL_BYTES / (cal_f * 1024), CAL_BYTES / (cal_w * 1024)
    rows = ["# Roofline of one forward, " + workload, "", f"Command: `{command}`", "",
            f"Peaks: MFMA {R.PEAK_MFMA_TFLOPS[w.dtype]:.0f} TFLOP/s ({synth.DTYPE_NAMES[w.dtype]}), HBM "
            f"{R.PEAK_HBM_GBS:.0f} GB/s.  HBM bytes = FETCH_SIZE x {ff:.3f} + WRITE_SIZE x {wf:.3f} (a {CAL_BYTES >> 20} MiB "
            "device copy reads those factors).  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x "
            "GRBM_GUI_ACTIVE / 8 XCDs).  A kernel class launched as several kernels sums them per launch.", "",
            "| kernel class | kernels | avg us / launch | work / launch | achieved | % of peak | HBM bytes / launch (measured) | measured GB/s | MFMA busy |",
            "|---|---|---|---|---|---|---|---|---|"]
    for kind, rx in R.KIND_REGEX.items():
        names = [r["Name"] for r in stats if _re.search(rx, r["Name"])]
        if not names:
            continue
        avg_us = sum(float(r["AverageNs"]) for r in stats if r["Name"] in names) / 1e3
        try:
            hbm = _one(fetch_csv, "FETCH_SIZE", rx) * 1024 * ff + _one(write_csv, "WRITE_SIZE", rx) * 1024 * wf
        except SystemExit:
            hbm = float("nan")
        busy = float("nan")
        try:
            mb = _one(sq_csv, "SQ_VALU_MFMA_BUSY_CYCLES", rx)
            ga = _one(sq_csv, "GRBM_GUI_ACTIVE", rx)
            busy = mb / (N_SIMD * ga / N_XCD)
        except SystemExit:
            pass
        if kind in R.MFMA_KINDS and not (kind == "embed" and "embed_kernel" in " ".join(names)):
            f = flops[kind]
            ach = f / (avg_us * 1e-6) / 1e12
            work, achs, frac = f"{f / 1e9:.1f} GFLOP", f"{ach:.0f} TFLOP/s", ach / R.PEAK_MFMA_TFLOPS[w.dtype]
        else:
            bb = byts.get(kind, float("nan"))
            ach = bb / (avg_us * 1e-6) / 1e9
            work, achs, frac = f"{bb / 1e6:.1f} MB", f"{ach:.0f} GB/s", ach / R.PEAK_HBM_GBS
        rows.append(f"| {kind} | {len(names)} | {avg_us:.1f} | {work} | {achs} | {100 * frac:.1f}% | {hbm / 1e6:.1f} MB | "
                    f"{hbm / (avg_us * 1e-6) / 1e9:.0f} | {100 * busy:.1f}% |")
    return "\n".join(rows) + "\n"


def waves_md(pass1_csv, pass2_csv, workload, command) -> str:
    """Where each kernel class's waves spend their cycles, from two counter passes over the same
    program: fractions of SQ_WAVE_CYCLES (busy, waiting on a counter, waiting to issue, issuing any /
    vector-and-matrix / LDS instructions, waiting on LDS), LDS bank-conflict cycles per LDS
    instruction, vector instructions per matrix instruction, and the matrix-core busy fraction."""
    sys.path.insert(0, os.path.dirname(HERE))
    from axial_band_split_amd import roofline as R
    rows = ["# Where the waves spend their cycles (" + workload + ")", "", f"Command: `{command}`", "",
            "Fractions of SQ_WAVE_CYCLES per kernel class (mean per dispatch, summed over the class's kernels); "
            "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs).", "",
            "| kernel class | busy | wait (any) | wait for issue | issuing any | issuing VALU+MFMA | issuing LDS | "
            "waiting on LDS | LDS bank-conflict cycles / LDS instr | VALU / MFMA instr | MFMA busy |",
            "|---|---|---|---|---|---|---|---|---|---|---|"]
    for kind, rx in R.KIND_REGEX.items():
        try:
            wc = _one(pass1_csv, "SQ_WAVE_CYCLES", rx)
        except SystemExit:
            continue
        g1 = lambda c: _one(pass1_csv, c, rx)
        g2 = lambda c: _one(pass2_csv, c, rx)
        try:
            mfma = g2("SQ_INSTS_MFMA")
            ratio = g2("SQ_INSTS_VALU") / mfma if mfma else float("nan")
            busy = g2("SQ_VALU_MFMA_BUSY_CYCLES") / (N_SIMD * g2("GRBM_GUI_ACTIVE") / N_XCD)
            act_any, act_valu = g2("SQ_ACTIVE_INST_ANY") / wc, g2("SQ_ACTIVE_INST_VALU") / wc
        except SystemExit:
            ratio = busy = act_any = act_valu = float("nan")
        lds = g1("SQ_INSTS_LDS")
        conf = g1("SQ_LDS_BANK_CONFLICT") / lds if lds else 0.0
        rows.append(f"| {kind} | {g1('SQ_BUSY_CYCLES') / wc:.2f} | {g1('SQ_WAIT_ANY') / wc:.2f} | "
                    f"{g1('SQ_WAIT_INST_ANY') / wc:.2f} | {act_any:.2f} | {act_valu:.2f} | {g1('SQ_ACTIVE_INST_LDS') / wc:.2f} | "
                    f"{g1('SQ_WAIT_INST_LDS') / wc:.2f} | {conf:.2f} | {ratio:.1f} | {100 * busy:.0f}% |")
    return "\n".join(rows) + "\n"


def sweep_md(paths, command) -> str:
    """One row per bench line: the workload's shape, throughput and the per-kernel device time."""
    recs = [json.loads(open(p).read().strip().splitlines()[-1]) for p in paths]
    kinds = []
    for r in recs:
        for k in r["kernels"]:
            if k not in kinds:
                kinds.append(k)
    lines = ["# Throughput against the workload's shape", "", f"Commands: `{command}`", "",
             "| workload | B | T | stems | ms / step | audio-s/s | attn+GEMM TFLOP/s | " + " | ".join(f"{k} ms" for k in kinds) + " |",
             "|---|---|---|---|---|---|---|" + "---|" * len(kinds)]
    for r in recs:
        c = r["config"]
        lines.append(f"| {c['workload']} | {c['batch']} | {c['frames']} | {c.get('stems', 1)} | {r['ms_per_step']:.3f} | "
                     f"{r['value']:.1f} | {r['attn_gemm']['tflops']:.0f} | "
                     + " | ".join(f"{r['kernels'][k]['ms_per_step']:.3f}" if k in r["kernels"] else "-" for k in kinds) + " |")
    return "\n".join(lines) + "\n"


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
    e = sub.add_parser("sweep")
    e.add_argument("paths", nargs="+")
    e.add_argument("--command", required=True)
    f = sub.add_parser("waves")
    for n in ("pass1", "pass2", "workload", "out"):
        f.add_argument(n)
    f.add_argument("--command", required=True)
    d = sub.add_parser("roofline")
    for n in ("stats", "fetch", "write", "cal_fetch", "cal_write", "sq", "workload", "out"):
        d.add_argument(n)
    d.add_argument("--command", required=True)
    args = ap.parse_args(argv)
    if args.what == "calibrate":
        calibrate()
        return 0
    if args.what == "sweep":
        open(args.paths[-1], "w").write(sweep_md(args.paths[:-1], args.command))
        return 0
    if args.what == "waves":
        open(args.out, "w").write(waves_md(args.pass1, args.pass2, args.workload, args.command))
        return 0
    if args.what == "roofline":
        open(args.out, "w").write(roofline_md(args.stats, args.fetch, args.write, args.cal_fetch, args.cal_write,
                                              args.sq, args.workload, args.command))
        return 0
    if args.what == "stats":
        open(args.out, "w").write(stats_md(args.csv, args.command))
    elif args.what == "counters":
        open(args.out, "w").write(counters_md(args.csv, args.command))
    else:
        sys.path.insert(0, os.path.dirname(HERE))
        from axial_band_split_amd import roofline as R
        kind = next((k for k, v in R.KIND_REGEX.items() if v == args.regex), None)
        rec = traffic_record(args.fetch, args.write, args.cal_fetch, args.cal_write, args.regex, args.command,
                             KIND_SOURCES.get(kind))
        json.dump(rec, open(args.out, "w"), indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
