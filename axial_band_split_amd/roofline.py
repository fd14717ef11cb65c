"""Algorithmic work of the core's kernels, for throughput and roofline reporting.

FLOPs follow the convention of [P1] section "FLOP shares": multiply-accumulates of every linear
layer and of the two attention products (q k^T and p v), FLOPs = 2 x MACs, nothing for softmax,
norms or activations.  Bytes of the memory-bound passes are the minimal traffic: each input read
once and each output written once.

MI355X peaks (AMD's published dense figures): HBM 8 TB/s; MFMA fp16 / bf16 2.5 PFLOP/s, fp32
157.3 TFLOP/s.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict

from . import synth

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = {synth.F32: 157.3, synth.F16: 2500.0, synth.BF16: 2500.0}


@dataclass
class Shape:
    B: int
    T: int
    NB: int
    D: int
    H: int
    dh: int
    FF: int
    MH: int
    total_width: int      # sum of band input widths
    depth: int
    mask_depth: int
    stems: int
    n_freqs: int
    channels: int
    esz: int              # bytes per operand element

    @property
    def tokens(self) -> int:
        return self.NB * self.B * self.T

    @property
    def inner(self) -> int:
        return self.H * self.dh


def shape_of(w: synth.Workload, total_width: int, batch: int | None = None) -> Shape:
    return Shape(B=w.batch if batch is None else batch, T=w.frames, NB=w.num_bands, D=w.dim, H=w.heads,
                 dh=w.dim_head, FF=w.ff_mult * w.dim, MH=w.mask_hidden_mult * w.dim, total_width=total_width,
                 depth=w.depth, mask_depth=w.mask_depth, stems=w.num_stems, n_freqs=w.freqs,
                 channels=w.audio_channels, esz=4 if w.dtype == synth.F32 else 2)


# rocprofv3 kernel-name patterns of each kernel class on the 16-bit path (the GEMM's epilogue id is
# its second template argument)
KIND_REGEX = {"embed": r"gemm2_kernelIDF16b?_?Li0E|embed_kernel", "qkv": r"gemm2_kernelIDF16b?_?Li1E|gemm2_kernel<bool _Accum, int, E,",
              "ffn1": r"gemm2_kernelIDF16b?_?Li2E", "out_proj": r"gemm2_kernelIDF16b?_?Li3E",
              "mask_hidden": r"gemm2_kernelIDF16b?_?Li4E", "mask_glu": r"gemm2_kernelIDF16b?_?Li5E",
              "ffn2": r"gemm2_kernelIDF16b?_?Li7E", "attn_time": r"attn_time2", "attn_band": r"attn_band",
              "norm": r"norm", "gather": r"gather", "average": r"average",
              "block": r"block_kernel|block_reduce_kernel", "band_attn": r"band_attn_kernel"}
MFMA_KINDS = ("embed", "qkv", "attn_time", "out_proj", "ffn1", "ffn2", "mask_hidden", "mask_glu", "block",
              "band_attn")
HBM_KINDS = ("gather", "average", "attn_band", "norm")


def flops_per_launch(s: Shape) -> Dict[str, float]:
    """FLOPs of one launch of each kernel class (per Transformer for the trunk kernels)."""
    N, D, I, H = s.tokens, s.D, s.inner, s.H
    BT = s.B * s.T
    return {
        "embed": 2.0 * BT * D * s.total_width,
        "norm_gates": 2.0 * N * D * H,                       # gate projection inside the norm pass
        "qkv": 2.0 * N * D * 3 * I,
        "attn_time": 2.0 * 2.0 * (s.NB * s.B) * H * s.T * s.T * s.dh,
        "attn_band": 2.0 * 2.0 * BT * H * s.NB * s.NB * s.dh,
        "out_proj": 2.0 * N * I * D,
        "ffn1": 2.0 * N * D * s.FF,
        "ffn2": 2.0 * N * s.FF * D,
        # the mask head: one launch per layer covers every stem
        "mask_hidden_first": 2.0 * s.stems * BT * s.NB * D * s.MH,
        "mask_hidden_next": 2.0 * s.stems * BT * s.NB * s.MH * s.MH,
        "mask_glu": 2.0 * s.stems * BT * s.MH * 2 * s.total_width,
        # out-projection + feed-forward of one Transformer in one kernel (16-bit path)
        "block": 2.0 * N * I * D + 4.0 * N * D * s.FF,
        # the band axis' q, k, v projection and attention in one kernel (16-bit path)
        "band_attn": 2.0 * N * D * 3 * I + 2.0 * 2.0 * BT * H * s.NB * s.NB * s.dh,
    }


def flops_forward(s: Shape) -> Dict[str, float]:
    """FLOPs of a whole forward by part (trunk counts both axes of every layer)."""
    f = flops_per_launch(s)
    L = s.depth
    per_axis = f["qkv"] + f["norm_gates"] + f["out_proj"] + f["ffn1"] + f["ffn2"]
    trunk = 2 * L * per_axis + L * (f["attn_time"] + f["attn_band"])
    mask = f["mask_hidden_first"] + (s.mask_depth - 1) * f["mask_hidden_next"] + f["mask_glu"]
    return {"embed": f["embed"], "trunk": trunk, "mask": mask, "total": f["embed"] + trunk + mask,
            "attn": L * (f["attn_time"] + f["attn_band"])}


def bytes_per_launch(s: Shape) -> Dict[str, float]:
    """Minimal HBM bytes of one launch of each memory-bound pass."""
    N, D = s.tokens, s.D
    BT = s.B * s.T
    spec = 4.0 * BT * s.n_freqs * s.channels * 2
    return {
        "gather": spec + BT * s.total_width * s.esz,
        # band gather and embedding in one kernel (16-bit path): the spectrum read once, x0 written in
        # fp32 and in 16 bits
        "embed": spec + N * D * 4.0 + N * D * s.esz,
        "norm_pre": N * D * 4.0 + N * D * s.esz,                 # read x, write x^
        "norm_out": N * D * 4.0 * 2 + N * D * s.esz,             # read x, write x and x^
        "average": 4.0 * s.stems * BT * s.total_width + s.stems * spec,
        "attn_band": 4.0 * N * s.inner * s.esz,                   # q, k, v read, o written
        # fused post-attention kernel: o read, x read and written (fp32), x^ written, weights once
        "block": N * s.inner * s.esz + N * D * 8.0 + N * D * s.esz
                 + (s.inner / 64 + s.FF / 32 + 2) * D * 64 * s.esz,
    }
