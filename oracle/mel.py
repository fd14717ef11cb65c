"""Mel band tables of the Mel-Band RoFormer core (oracle side, fp64, test infrastructure).

[P1] section "The mel-band split, exactly": a Slaney-mel triangular filter bank
(librosa's defaults: fmin 0, fmax sr/2) with n_mels = number of bands over the
n_fft/2+1 STFT bins is binarised (weight > 0); entry [0][0] (DC into the first
band) and [-1][-1] (Nyquist into the last band) are forced to 1; each band keeps its
bins in ascending order with the stereo channels interleaved (pair = bin*S + s).
The per-bin band count divides the scatter-added masks ("num_bands_per_freq").
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List

import numpy as np

# Slaney's mel scale: linear (200/3 Hz per mel) below 1 kHz, logarithmic above, with
# 27 mels per factor 6.4 in frequency.
_F_SP = 200.0 / 3.0
_MIN_LOG_HZ = 1000.0
_MIN_LOG_MEL = _MIN_LOG_HZ / _F_SP
_LOGSTEP = math.log(6.4) / 27.0


def hz_to_mel(f):
    f = np.asarray(f, dtype=np.float64)
    lin = f / _F_SP
    log = _MIN_LOG_MEL + np.log(np.maximum(f, _MIN_LOG_HZ) / _MIN_LOG_HZ) / _LOGSTEP
    return np.where(f >= _MIN_LOG_HZ, log, lin)


def mel_to_hz(m):
    m = np.asarray(m, dtype=np.float64)
    lin = _F_SP * m
    log = _MIN_LOG_HZ * np.exp(_LOGSTEP * (np.maximum(m, _MIN_LOG_MEL) - _MIN_LOG_MEL))
    return np.where(m >= _MIN_LOG_MEL, log, lin)


def filter_bank(sample_rate: int, n_fft: int, n_mels: int) -> np.ndarray:
    """Triangular Slaney mel weights [n_mels, n_fft//2+1] (without the area normalisation,
    a positive per-row scale that does not change which weights are > 0)."""
    n_freqs = n_fft // 2 + 1
    fft_hz = np.linspace(0.0, sample_rate / 2.0, n_freqs)
    mel_pts = np.linspace(hz_to_mel(0.0), hz_to_mel(sample_rate / 2.0), n_mels + 2)
    hz_pts = mel_to_hz(mel_pts)
    w = np.zeros((n_mels, n_freqs))
    for i in range(n_mels):
        lo, mid, hi = hz_pts[i], hz_pts[i + 1], hz_pts[i + 2]
        rising = (fft_hz - lo) / (mid - lo)
        falling = (hi - fft_hz) / (hi - mid)
        w[i] = np.maximum(0.0, np.minimum(rising, falling))
    return w


def incidence(sample_rate: int, n_fft: int, n_mels: int) -> np.ndarray:
    """Binarised filter bank with DC forced into band 0 and Nyquist into the last band."""
    inc = filter_bank(sample_rate, n_fft, n_mels) > 0.0
    inc[0, 0] = True
    inc[-1, -1] = True
    return inc


@dataclass
class BandTables:
    n_freqs: int
    channels: int
    bins: List[np.ndarray]          # per band: ascending bin indices
    pairs: List[np.ndarray]         # per band: pair indices bin*S + s, bin-major, stereo-minor
    widths: np.ndarray              # per band: input width W_i = 2 * S * |bins_i|
    counts: np.ndarray              # per bin: number of bands covering it
    incidence: np.ndarray           # [bands, n_freqs] bool

    @property
    def num_bands(self) -> int:
        return len(self.bins)

    @property
    def total_width(self) -> int:
        return int(self.widths.sum())

    def feature_offsets(self) -> np.ndarray:
        """Start of each band's features in the concatenation of all bands' features."""
        return np.concatenate([[0], np.cumsum(self.widths)[:-1]]).astype(np.int64)


def band_tables(sample_rate: int, n_fft: int, n_mels: int, channels: int) -> BandTables:
    inc = incidence(sample_rate, n_fft, n_mels)
    n_freqs = inc.shape[1]
    if not inc.any(axis=0).all():
        raise ValueError("a frequency bin is covered by no band")
    bins = [np.nonzero(inc[i])[0].astype(np.int64) for i in range(n_mels)]
    pairs = [(b[:, None] * channels + np.arange(channels)[None, :]).reshape(-1) for b in bins]
    widths = np.array([2 * channels * len(b) for b in bins], dtype=np.int64)
    counts = inc.sum(axis=0).astype(np.int64)
    return BandTables(n_freqs, channels, bins, pairs, widths, counts, inc)


def explicit_band_tables(n_fft: int, band_bins, channels: int) -> BandTables:
    """Contiguous, non-overlapping bands given by their bin counts, low to high, covering every
    bin once (the band-split table kind: [P2] "Evaluation record", the BS PolarFormer section, a
    62-band table over all 1025 bins)."""
    n_freqs = n_fft // 2 + 1
    band_bins = [int(n) for n in band_bins]
    if min(band_bins) < 1 or sum(band_bins) != n_freqs:
        raise ValueError("band bin counts must be >= 1 and add up to n_fft/2 + 1")
    starts = np.concatenate([[0], np.cumsum(band_bins)[:-1]])
    inc = np.zeros((len(band_bins), n_freqs), dtype=bool)
    for i, (k0, n) in enumerate(zip(starts, band_bins)):
        inc[i, k0:k0 + n] = True
    bins = [np.nonzero(inc[i])[0].astype(np.int64) for i in range(len(band_bins))]
    pairs = [(b[:, None] * channels + np.arange(channels)[None, :]).reshape(-1) for b in bins]
    widths = np.array([2 * channels * len(b) for b in bins], dtype=np.int64)
    return BandTables(n_freqs, channels, bins, pairs, widths, inc.sum(axis=0).astype(np.int64), inc)


def stft_frames(num_samples: int, hop: int) -> int:
    """Frames of a centred STFT ([P1] "The two transformers are not the same shape": 1 + samples/hop)."""
    return 1 + num_samples // hop
