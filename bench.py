#!/usr/bin/env python3
"""Throughput of the Mel-Band RoFormer core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload chunk11s_fp16]

A step is one forward of the whole core (band gather and embedding, every axial Transformer, the
mask head, the mask average) over one batch of seeded synthetic spectra already resident in HBM.
Prints one JSON line: core audio-seconds per second, the median / p10 / p90 of single forwards
and the per-kernel device times (HIP events on the launch stream), the roofline of the dominant kernel, the fp64 CPU oracle timed on
a bounded sample of the same workload, and (beside the headline figure) the separation of a
synthetic 60 s stereo track through STFT, core, iSTFT and the chunked overlap-add.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from axial_band_split_amd import binding, roofline, synth  # noqa: E402

METRIC = "core audio-seconds/sec (44.1 kHz stereo) at T=1100; attn+GEMM TFLOP/s vs peak"
KIND_REGEX = roofline.KIND_REGEX
MFMA_KINDS = roofline.MFMA_KINDS
GEMM_ATTN_KINDS = MFMA_KINDS + ("attn_band",)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_for(workload: str, kind: str):
    """HBM bytes per launch of a kernel class from the committed counter record, or None when there
    is no record for it or the kernel sources changed since it was taken."""
    from axial_band_split_amd import profiling
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_regex") != KIND_REGEX.get(kind) or rec.get("source_sha") != profiling.source_hash(rec.get("source_files")):
        return None
    return rec["bytes_per_launch"]


def kind_flops(s: roofline.Shape, kind: str, w: synth.Workload) -> float:
    f = roofline.flops_per_launch(s)
    if kind == "mask_hidden":   # average over the hidden layers of a stem
        return (f["mask_hidden_first"] + (w.mask_depth - 1) * f["mask_hidden_next"]) / w.mask_depth
    return f[kind]


def cpu_baseline(w: synth.Workload, ws, x_io, flops: float) -> dict:
    """The oracle on a bounded sample of the same workload.  Up to 6 TFLOP per forward (the 11 s
    chunk at depth 6 is 4.5, about half a minute on the host's cores) the whole oracle forward is
    timed once; a larger forward is estimated from its parts, each timed once: the band embedding,
    the time and band Transformers of the first layers (up to three), the mask head and the average,
    as embedding + depth x (mean layer) + stems x (mask head + average), since every layer has the
    same shape and cost."""
    from oracle import model as M

    cfg = M.CoreConfig(w.sample_rate, w.n_fft, w.audio_channels, w.num_bands, w.dim, w.depth, w.heads,
                       w.dim_head, w.ff_mult, w.mask_hidden_mult, w.mask_depth, w.num_stems)
    if flops <= 6e12:
        t0 = time.perf_counter()
        M.forward(x_io, cfg, ws, layout=w.io_layout)
        t3 = time.perf_counter()
        est = t3 - t0
        sample = (f"one whole fp64 numpy oracle forward of {w.name} ({w.audio_seconds:g} s of audio, every layer "
                  f"and the mask head), timed once: {est:.1f} s")
    else:
        tables = cfg.tables()
        wn = M.named(cfg, ws)
        spec = M.read_input(x_io, w.audio_channels, w.io_layout)
        layers = min(w.depth, 3)
        t0 = time.perf_counter()
        x = M.band_embed(spec, cfg, wn, tables)
        t1 = time.perf_counter()
        for i in range(layers):
            x = M.time_transformer(x, cfg, wn, f"layer{i}.time.", chunk=1)
            x = M.band_transformer(x, cfg, wn, f"layer{i}.band.", chunk=64)
        t2 = time.perf_counter()
        m = M.mask_head(x, cfg, wn, tables, 0)
        M.average(m, tables)
        t3 = time.perf_counter()
        est = (t1 - t0) + w.depth * (t2 - t1) / layers + w.num_stems * (t3 - t2)
        sample = (f"fp64 numpy oracle on {w.name}: band embedding, {layers} of {w.depth} layers (time + band "
                  f"Transformer), mask head and average of stem 0, each timed once ({t3 - t0:.1f} s); "
                  f"forward estimated as embed + {w.depth} x mean layer + {w.num_stems} x mask head = {est:.1f} s")
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info())
    except Exception:
        pass
    cores = max(threads or 1, M._WORKERS)
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{b.get('name')} {b.get('version')}"
    except Exception:
        blas = None
    return {"value": w.audio_seconds / est, "unit": "audio-s/s", "cores": cores, "kind": "oracle",
            "sample": sample, "host_cpus": os.cpu_count(), "blas": blas, "blas_threads": threads,
            "seconds_sampled": t3 - t0}


def separation(w: synth.Workload, ws, seconds: float, repeats: int) -> dict:
    """A whole track through the separation entry point: chunked STFT, the core over all chunks at
    once (max_batch = the chunk count), masks x STFT, inverse STFT, faded overlap-add.  Input resident
    in HBM; wall time of `repeats` calls after one warm call, synchronised on both sides."""
    import torch
    hop = w.hop
    L = int(seconds * w.sample_rate)
    chunk = (w.frames - 1) * hop
    stride = int(chunk * 0.9)
    pad = chunk - stride if L > 2 * (chunk - stride) else 0
    n_chunks = -(-(L + 2 * pad) // stride)
    cfg = binding.config(w, max_batch=n_chunks)
    core = binding.Core(cfg, ws)
    wave = torch.from_numpy(synth.draw_wave(w.audio_channels, L, seed=w.input_seed)).cuda()
    core.separate(wave, hop)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(repeats):
        y = core.separate(wave, hop)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ok = bool(torch.isfinite(y).all().item())
    core.close()
    ms = (t1 - t0) * 1e3 / repeats
    return {"track_seconds": L / w.sample_rate, "chunk_samples": chunk, "stride_samples": stride, "chunks": n_chunks,
            "max_batch": n_chunks, "repeats": repeats, "ms_per_track": ms, "audio_s_per_s": L / w.sample_rate / (ms * 1e-3),
            "finite": ok}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="chunk11s_fp16", choices=list(synth.WORKLOADS))
    ap.add_argument("--frames", type=int, default=0, help="override the workload's frames per chunk")
    ap.add_argument("--stems", type=int, default=0, help="override the number of mask heads")
    ap.add_argument("--batch", type=int, default=0, help="override the chunks per call")
    ap.add_argument("--profile-steps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-seconds", type=float, default=60.0,
                    help="also time the separation of a synthetic track of this length (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; the core runs on one GPU (no sharding, no "
              f"collectives). Run with --gpus 1.", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1

    w = synth.WORKLOADS[args.workload]
    over = {k: v for k, v in (("frames", args.frames), ("num_stems", args.stems), ("batch", args.batch)) if v}
    if over:
        w = w.replace(**over, name=w.name + "".join(f"@{k}={v}" for k, v in over.items()))
    log(f"[bench] workload {w.name}: B={w.batch} T={w.frames} D={w.dim} depth={w.depth} "
        f"dtype={synth.DTYPE_NAMES[w.dtype]}")
    cfg = binding.config(w)
    inv = binding.inventory(cfg)
    _, total_width, _ = binding.mbr_core_table_sizes(cfg)
    ws = synth.draw_weights(inv, w.dtype, seed=w.weight_seed)
    x_np = synth.input_in_layout(w, synth.draw_input(w))
    core = binding.Core(cfg, ws)
    log(f"[bench] core created: {core.device_bytes() / 2**30:.2f} GiB on the device")
    x = torch.from_numpy(x_np).cuda()
    out = torch.empty(core.output_shape(w.batch), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        core.forward(x, out, stream)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        core.forward(x, out, stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = w.audio_seconds * args.steps / (t1 - t0)
    log(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step, {value:.1f} audio-s/s")

    # spread of single forwards: an event pair on the launch stream around each one (after the
    # timed region, so the events cost it nothing)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record(stream)
        core.forward(x, out, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    q = lambda f: per[min(len(per) - 1, int(round(f * (len(per) - 1))))]
    spread = {"median": q(0.5), "p10": q(0.1), "p90": q(0.9), "forwards": len(per)}
    log(f"[bench] single forwards: median {spread['median']:.3f} ms, p10 {spread['p10']:.3f}, p90 {spread['p90']:.3f}")

    # per-kernel device time: HIP event pairs around every launch on the launch stream
    acc = {k: [0.0, 0] for k in binding.KERNEL_KINDS}
    tp0 = time.perf_counter()
    for _ in range(args.profile_steps):
        prof = core.profile(x, out, stream)
        for k, (ms, n) in prof.items():
            acc[k][0] += ms
            acc[k][1] += n
    tp1 = time.perf_counter()
    P = args.profile_steps
    s = roofline.shape_of(w, total_width)
    fl = roofline.flops_forward(s)
    kernels = {}
    for k, (ms, n) in acc.items():
        if n == 0:
            continue
        e = {"ms_per_step": ms / P, "launches_per_step": n // P, "avg_launch_ms": ms / n}
        if k in MFMA_KINDS or k == "attn_band":
            e["tflops"] = kind_flops(s, k, w) / (ms / n * 1e-3) / 1e12
        kernels[k] = e
    dev_ms = sum(v["ms_per_step"] for v in kernels.values())
    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dominant]
    peak_mfma = roofline.PEAK_MFMA_TFLOPS[w.dtype]
    if dominant in MFMA_KINDS:
        ach = kind_flops(s, dominant, w) / (dk["avg_launch_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dominant, "achieved": ach, "peak": peak_mfma, "unit": "TFLOP/s",
                "frac": ach / peak_mfma, "traffic": traffic_for(w.name, dominant),
                "flops_per_launch": kind_flops(s, dominant, w), "avg_launch_ms": dk["avg_launch_ms"]}
    else:
        b = roofline.bytes_per_launch(s)
        key = {"norm": "norm_pre", "gather": "gather", "average": "average", "attn_band": "attn_band"}[dominant]
        ach = b[key] / (dk["avg_launch_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dominant, "achieved": ach, "peak": roofline.PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / roofline.PEAK_HBM_GBS, "traffic": traffic_for(w.name, dominant), "bytes_per_launch": b[key],
                "avg_launch_ms": dk["avg_launch_ms"]}
    ga_ms = sum(kernels[k]["ms_per_step"] for k in GEMM_ATTN_KINDS if k in kernels)
    ga_tflops = fl["total"] / (ga_ms * 1e-3) / 1e12
    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["ms_per_step"]):
        log(f"[bench]   {k:12s} {v['ms_per_step']:8.3f} ms/step  {v['launches_per_step']:4d} launches"
            + (f"  {v['tflops']:7.1f} TFLOP/s" if "tflops" in v else ""))

    sep = None
    if args.separate_seconds > 0 and w.io_layout == synth.IO_FS_T_C:
        sep = separation(w, ws, args.separate_seconds, 5)
        log(f"[bench] separation of {sep['track_seconds']:.0f} s in {sep['chunks']} chunks: {sep['ms_per_track']:.2f} ms, "
            f"{sep['audio_s_per_s']:.1f} audio-s/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle, bounded sample) ...")
        cpu = cpu_baseline(w, ws, x_np, fl["total"])
        log(f"[bench] cpu baseline: {cpu['value']:.4f} audio-s/s ({cpu['sample']})")

    line = {
        "metric": METRIC if w.frames == 1100 else METRIC.replace("T=1100", f"T={w.frames}"), "value": value, "unit": "audio-s/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": synth.DTYPE_NAMES[w.dtype], "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "frames": w.frames, "stems": w.num_stems,
                   "bands": w.num_bands, "dim": w.dim,
                   "depth": w.depth, "heads": w.heads, "dim_head": w.dim_head, "io_layout": w.io_layout,
                   "audio_seconds_per_step": w.audio_seconds},
        "roofline": roof,
        "cpu_baseline": cpu,
        "attn_gemm": {"tflops": ga_tflops, "peak": peak_mfma, "frac": ga_tflops / peak_mfma,
                      "flops_per_step": fl["total"], "device_ms": ga_ms},
        "e2e_tflops": fl["total"] / (ms_step * 1e-3) / 1e12,
        "forward_ms": spread,
        "device_ms_per_step": dev_ms,
        "profiled_ms_per_step": (tp1 - tp0) * 1e3 / P,
        "kernels": kernels,
        "separation": sep,
    }
    core.close()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
