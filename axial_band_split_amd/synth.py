"""Seeded synthetic workloads: the five core configurations and their inputs and weights.

This module only describes sizes and draws random numbers.  It holds none of the
method's arithmetic (no band tables, no norms, no layers): both the HIP path and
the oracle receive the arrays made here, so parity compares the two on
identical inputs.

Inputs follow the shapes the pages run the core at:
  * "Mel-Band RoFormer — architecture, inference hot path & RTX 3050 feasibility",
    section "Architecture / The forward chain": the complex stereo STFT merged into
    the frequency axis, (B, F*S, T, 2), 801 frames for an 8 s chunk;
  * "Vocal Separation Core (Mel-Band RoFormer) — ONNX / fp16 / WebGPU", section
    "How to use" / signature table: stft_repr float32 [1, 2050, T, 2], T = 1100;
  * "Mel-Band RoFormer (vocals), ONNX for the GPU", section "Graph": mix_spec
    [1, 4, 1025, 801] with planes L re, L im, R re, R im.

No public data set stands behind these shapes here: the spectra are drawn with a
1/f magnitude and uniform phase so that no band is silent (the pages warn that
a silent band turns rounding into its direction once each band is normalised).
"""
from __future__ import annotations

import dataclasses
from typing import Iterable, List, Sequence, Tuple

import numpy as np

# dtype codes shared with the C header (MBR_F32 / MBR_F16 / MBR_BF16)
F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
# io layouts (MBR_IO_FS_T_C / MBR_IO_SC_F_T)
IO_FS_T_C, IO_SC_F_T = 0, 1
# weight kinds in an inventory: a matrix, a bias vector, an RMSNorm gain
KIND_MATRIX, KIND_BIAS, KIND_GAMMA = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    sample_rate: int
    n_fft: int
    audio_channels: int
    num_bands: int
    frames: int
    batch: int
    dim: int
    depth: int
    heads: int
    dim_head: int
    ff_mult: int
    mask_hidden_mult: int
    mask_depth: int
    num_stems: int
    dtype: int
    io_layout: int
    input_kind: str          # "normal" (re, im iid N(0,1)) or "one_over_f"
    weight_seed: int
    input_seed: int
    hop: int = 441
    zero_dc: int = 0
    band_bins: Tuple[int, ...] | None = None   # explicit non-overlapping band table (None: mel)

    @property
    def freqs(self) -> int:
        return self.n_fft // 2 + 1

    @property
    def audio_seconds(self) -> float:
        """Audio covered by one call: B chunks of T frames at hop/sr seconds a frame."""
        return self.batch * self.frames * self.hop / self.sample_rate

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # 8 bands at n_fft 256, 32 frames, D=64, one layer of 2 heads x 32: the oracle's small case
    "tiny_fp32": Workload("tiny_fp32", 44100, 256, 2, 8, 32, 1, 64, 1, 2, 32, 4, 4, 2, 1,
                          F32, IO_FS_T_C, "normal", 0, 0),
    # the vocals model (60 bands, D=384, depth 6, 8 x 64 heads) at 256 frames
    "t256_fp16": Workload("t256_fp16", 44100, 2048, 2, 60, 256, 1, 384, 6, 8, 64, 4, 4, 2, 1,
                          F16, IO_FS_T_C, "one_over_f", 0, 2),
    # one 8 s chunk (801 frames), input in the [B, S*2, F, T] plane layout
    "chunk8s_bf16": Workload("chunk8s_bf16", 44100, 2048, 2, 60, 801, 1, 384, 6, 8, 64, 4, 4, 2, 1,
                             BF16, IO_SC_F_T, "one_over_f", 0, 3),
    # one 11 s chunk (1100 frames)
    "chunk11s_fp16": Workload("chunk11s_fp16", 44100, 2048, 2, 60, 1100, 1, 384, 6, 8, 64, 4, 4, 2, 1,
                              F16, IO_FS_T_C, "one_over_f", 0, 4),
    # four 11 s chunks through a D=512, depth-12 model
    "heavy_b4_d512_bf16": Workload("heavy_b4_d512_bf16", 44100, 2048, 2, 60, 1100, 4, 512, 12, 8, 64, 4, 4, 2, 1,
                                   BF16, IO_FS_T_C, "one_over_f", 0, 5),
}
WORKLOAD_ORDER = list(WORKLOADS)


# ----------------------------------------------------------------------------- rounding

def round_to_dtype(a: np.ndarray, dtype: int) -> np.ndarray:
    """Round fp64 values once to the storage dtype (round to nearest even) and return
    them as float64 holding exactly the rounded values."""
    a = np.asarray(a, dtype=np.float64)
    if dtype == F32:
        return a.astype(np.float32).astype(np.float64)
    if dtype == F16:
        return a.astype(np.float16).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f64(f64_to_bf16_bits(a))
    raise ValueError(f"unknown dtype {dtype}")


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 bits (RNE on the upper 16 bits)."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32)).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7F800000) == 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r = np.where(nan & ((u & 0x7FFFFF) != 0), np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def storage_bytes(a: np.ndarray, dtype: int) -> np.ndarray:
    """The array in the library's storage format: float32, float16 or bf16 bit patterns."""
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == F16:
        return np.ascontiguousarray(a, dtype=np.float16)
    if dtype == BF16:
        return np.ascontiguousarray(f64_to_bf16_bits(a))
    raise ValueError(f"unknown dtype {dtype}")


# ----------------------------------------------------------------------------- weights

def draw_weights(inventory: Sequence[Tuple[str, Tuple[int, ...], int]], dtype: int, seed: int = 0,
                 std: float = 0.02, gamma_std: float = 0.02) -> List[np.ndarray]:
    """Draw every tensor of `inventory` in order from one generator.

    Matrices and biases: N(0, std).  RMSNorm gains: 1 + N(0, gamma_std) (the module
    initialises them to ones; the jitter makes a forgotten gain visible).  Each value
    is drawn in fp64 and rounded once to `dtype`; the returned fp64 arrays hold the
    rounded values, so both sides of a parity test see identical weights.
    """
    rng = np.random.default_rng(seed)
    out = []
    for _name, shape, kind in inventory:
        z = rng.standard_normal(size=tuple(shape))
        if kind == KIND_GAMMA:
            a = 1.0 + gamma_std * z
        else:
            a = std * z
        out.append(round_to_dtype(a, dtype))
    return out


# ----------------------------------------------------------------------------- inputs

def draw_input(w: Workload, batch: int | None = None, seed: int | None = None) -> np.ndarray:
    """The complex stereo spectrum as float32 [B, F*S, T, 2] (pair p = f*S + s; last axis re, im).

    "normal": re, im iid N(0, 1).
    "one_over_f": magnitude |l| / max(f, 1) with l ~ Laplace(0, 1), phase ~ U[0, 2 pi).
    """
    B = w.batch if batch is None else batch
    rng = np.random.default_rng(w.input_seed if seed is None else seed)
    F, S, T = w.freqs, w.audio_channels, w.frames
    if w.input_kind == "normal":
        x = rng.standard_normal(size=(B, F * S, T, 2))
    elif w.input_kind == "one_over_f":
        lap = rng.laplace(0.0, 1.0, size=(B, F, S, T))
        phase = rng.uniform(0.0, 2.0 * np.pi, size=(B, F, S, T))
        f = np.maximum(np.arange(F, dtype=np.float64), 1.0)[None, :, None, None]
        mag = np.abs(lap) / f
        x = np.stack([mag * np.cos(phase), mag * np.sin(phase)], axis=-1).reshape(B, F * S, T, 2)
    else:
        raise ValueError(w.input_kind)
    return np.ascontiguousarray(x, dtype=np.float32)


def fs_t_c_to_sc_f_t(x: np.ndarray, channels: int) -> np.ndarray:
    """[B, F*S, T, 2] -> [B, S*2, F, T] (planes: channel-major, then re/im), a pure relayout."""
    B, FS, T, _ = x.shape
    F = FS // channels
    return np.ascontiguousarray(x.reshape(B, F, channels, T, 2).transpose(0, 2, 4, 1, 3).reshape(B, channels * 2, F, T))


def input_in_layout(w: Workload, x_fs_t_c: np.ndarray) -> np.ndarray:
    return x_fs_t_c if w.io_layout == IO_FS_T_C else fs_t_c_to_sc_f_t(x_fs_t_c, w.audio_channels)


def draw_wave(channels: int, length: int, seed: int = 0) -> np.ndarray:
    """A synthetic track as float32 [channels, length]: Gaussian noise shaped to a 1/f power
    spectrum (1/sqrt(f) amplitude above 20 Hz at 44.1 kHz), the channels a common part plus a
    private one (correlation about 0.8), scaled to an RMS of 0.1."""
    rng = np.random.default_rng(seed)
    f = np.maximum(np.fft.rfftfreq(length, 1.0 / 44100.0), 20.0)
    shape = 1.0 / np.sqrt(f)

    def noise():
        z = np.fft.rfft(rng.standard_normal(length)) * shape
        return np.fft.irfft(z, n=length)

    common = noise()
    x = np.stack([common + 0.5 * noise() for _ in range(channels)])
    x *= 0.1 / np.sqrt(np.mean(x * x))
    return np.ascontiguousarray(x, dtype=np.float32)


def shapes_equal(a: Iterable, b: Iterable) -> bool:
    return [tuple(x) for x in a] == [tuple(x) for x in b]
