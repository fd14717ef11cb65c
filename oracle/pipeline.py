"""The steps on either side of the core, oracle side (numpy fp64, test infrastructure only).

[P1] "The forward chain": the waveform (B, 2, L) goes through a centred STFT (n_fft 2048, hop
441, a Hann window of 2048, reflect padding), the complex bins with the stereo channels merged
into the frequency axis are the core's input [B, F*S, T, 2]; the core's complex masks multiply
the original STFT and an inverse STFT returns one waveform per stem.
[P1] "Verified inference hot path" (chunk arithmetic, steps 3-9): a track is cut into chunks of
8 s with a stride of 0.9 chunk (or of half a chunk, the segmenting of [P4] "Graph"), reflect-
padded by the border (chunk - stride) on both sides when it is longer than two borders; each
chunk's estimate is weighted by a linear fade window (fade = chunk / 10, no fade-in on the first
chunk, no fade-out on the last), summed, divided by the summed window (clamped at 1e-8), and the
padding is cropped.  A tail shorter than a chunk is reflect-
padded when it holds more than half a chunk of audio, else zero-padded.

Readings where the text leaves a detail open (each also stated in the design notes):
  * the Hann window is the periodic one (w[n] = 1/2 - 1/2 cos(2 pi n / N)), the default of the
    STFT the pages call;
  * the inverse STFT divides the windowed overlap-add by the summed squared window at each sample
    and takes the real inverse transform of the one-sided spectrum (the imaginary parts of the DC
    and Nyquist bins are ignored);
  * "reflect" mirrors without repeating the edge sample (x[-1] = x[1]);
  * the last chunk is the last one the stride loop visits (offset + stride >= padded length).
The FFT is numpy's (a library primitive serving as one step).
"""
from __future__ import annotations

from typing import Callable

import numpy as np


def hann(n_fft: int) -> np.ndarray:
    k = np.arange(n_fft, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * k / n_fft)


def reflect_index(i: np.ndarray, n: int) -> np.ndarray:
    """Index into [0, n) of position i of a signal reflected about its ends (edge not repeated)."""
    if n == 1:
        return np.zeros_like(i)
    period = 2 * (n - 1)
    m = np.mod(i, period)
    return np.where(m < n, m, period - m)


def stft(x: np.ndarray, n_fft: int, hop: int) -> np.ndarray:
    """x [C, L] -> complex [C, n_fft/2 + 1, T], T = 1 + L // hop, centred with reflect padding."""
    C, L = x.shape
    T = 1 + L // hop
    w = hann(n_fft)
    pos = np.arange(T)[:, None] * hop + np.arange(n_fft)[None, :] - n_fft // 2     # [T, n_fft]
    frames = x[:, reflect_index(pos, L)] * w                                        # [C, T, n_fft]
    return np.transpose(np.fft.rfft(frames, axis=-1), (0, 2, 1))


def istft(z: np.ndarray, n_fft: int, hop: int, length: int) -> np.ndarray:
    """complex [C, n_fft/2 + 1, T] -> [C, length]: windowed overlap-add over the summed squared window."""
    C, F, T = z.shape
    w = hann(n_fft)
    frames = np.fft.irfft(np.transpose(z, (0, 2, 1)), n=n_fft, axis=-1) * w        # [C, T, n_fft]
    total = n_fft + hop * (T - 1)
    y = np.zeros((C, total))
    env = np.zeros(total)
    for t in range(T):
        y[:, t * hop:t * hop + n_fft] += frames[:, t]
        env[t * hop:t * hop + n_fft] += w * w
    start = n_fft // 2
    return y[:, start:start + length] / env[start:start + length]


def to_core_input(z: np.ndarray) -> np.ndarray:
    """complex [S, F, T] -> stft_repr [1, F*S, T, 2] (pair = f*S + s)."""
    S, F, T = z.shape
    zz = np.transpose(z, (1, 0, 2)).reshape(F * S, T)
    return np.ascontiguousarray(np.stack([zz.real, zz.imag], axis=-1)[None])


def apply_masks(z: np.ndarray, masks: np.ndarray) -> np.ndarray:
    """complex [S, F, T] times the core's masks [stems, F*S, T, 2] -> complex [stems, S, F, T]."""
    S, F, T = z.shape
    m = masks[..., 0] + 1j * masks[..., 1]                                           # [stems, F*S, T]
    m = np.transpose(m.reshape(masks.shape[0], F, S, T), (0, 2, 1, 3))
    return z[None] * m


def default_stride(chunk: int) -> int:
    """[P1] "Verified inference hot path" step 3: stride = int(0.9 chunk)."""
    return int(chunk * 0.9)


def chunk_plan(length: int, chunk: int, stride: int | None = None):
    """Chunk arithmetic: (padded length, border applied, [(offset, n_valid, tail_mode)]) where
    tail_mode is 'full', 'reflect' or 'zero'.  stride None: [P1]'s 0.9 chunk; [P4] "Graph" segments
    every half chunk (8 s every 4 s), with the same border = chunk - stride and fades."""
    stride = default_stride(chunk) if stride is None else stride
    border = chunk - stride
    pad = border if length > 2 * border else 0
    Lp = length + 2 * pad
    plan = []
    for off in range(0, Lp, stride):
        n = min(chunk, Lp - off)
        mode = "full" if n == chunk else ("reflect" if n > chunk // 2 else "zero")
        plan.append((off, n, mode))
    return Lp, pad, plan


def fade_window(chunk: int, first: bool, last: bool) -> np.ndarray:
    fade = chunk // 10
    w = np.ones(chunk)
    if not first:
        w[:fade] = np.linspace(0.0, 1.0, fade)
    if not last:
        w[-fade:] = np.linspace(1.0, 0.0, fade)
    return w


def separate(wave: np.ndarray, core: Callable[[np.ndarray], np.ndarray], n_fft: int, hop: int, chunk: int,
             stems: int, stride: int | None = None) -> np.ndarray:
    """wave [S, L] -> [stems, S, L]: chunked STFT -> core -> masks x STFT -> iSTFT -> faded overlap-add.
    `core` maps stft_repr [1, F*S, T, 2] to masks [stems, F*S, T, 2]."""
    S, L = wave.shape
    stride = default_stride(chunk) if stride is None else stride
    Lp, pad, plan = chunk_plan(L, chunk, stride)
    x = wave[:, reflect_index(np.arange(Lp) - pad, L)] if pad else wave
    out = np.zeros((stems, S, Lp))
    counter = np.zeros(Lp)
    for ci, (off, n, mode) in enumerate(plan):
        part = x[:, off:off + n]
        if mode == "reflect":
            part = part[:, reflect_index(np.arange(chunk), n)]
        elif mode == "zero":
            part = np.concatenate([part, np.zeros((S, chunk - n))], axis=1)
        z = stft(part, n_fft, hop)
        masks = core(to_core_input(z))
        y = apply_masks(z, masks)                                                   # [stems, S, F, T]
        est = np.stack([istft(y[s], n_fft, hop, chunk) for s in range(stems)])       # [stems, S, chunk]
        w = fade_window(chunk, ci == 0, off + stride >= Lp)
        out[:, :, off:off + n] += est[:, :, :n] * w[:n]
        counter[off:off + n] += w[:n]
    out = out / np.maximum(counter, 1e-8)
    return out[:, :, pad:pad + L] if pad else out
