"""Pins of the oracle's band tables against the printed band table and closed forms."""
import json
import math
import os

import numpy as np
import pytest

from oracle import brute, mel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_counts():
    rows = [l for l in open(os.path.join(GOLDEN, "melband_60_band_bins.txt")) if l.strip() and not l.startswith("#")]
    return [int(v) for l in rows for v in l.split()]


def test_band_bins_match_printed_table():
    t = mel.band_tables(44100, 2048, 60, 2)
    assert [len(b) for b in t.bins] == _golden_counts()


def test_coverage_and_widths_match_printed_totals():
    t = mel.band_tables(44100, 2048, 60, 2)
    assert sum(len(b) for b in t.bins) == 1979
    assert int((t.counts == 1).sum()) == 71
    assert int((t.counts == 2).sum()) == 954
    assert t.widths[0] == 28 and t.widths[-1] == 520 and t.total_width == 7916


@pytest.mark.parametrize("sr,n_fft,nb", [(44100, 2048, 60), (44100, 256, 8), (44100, 32, 3), (48000, 1024, 32),
                                         (44100, 4096, 64), (22050, 512, 16)])
def test_closed_form_membership_agrees(sr, n_fft, nb):
    """Thresholding evaluated triangles equals the strict-interval closed form."""
    t = mel.band_tables(sr, n_fft, nb, 2)
    assert [b.tolist() for b in t.bins] == brute.bands(sr, n_fft, nb)


@pytest.mark.parametrize("sr,n_fft,nb", [(44100, 2048, 60), (44100, 256, 8)])
def test_no_bin_sits_on_a_mel_point(sr, n_fft, nb):
    """The > 0 test is robust: every bin centre is clear of every mel point."""
    F = n_fft // 2 + 1
    pts = mel.mel_to_hz(np.linspace(mel.hz_to_mel(0.0), mel.hz_to_mel(sr / 2), nb + 2))[1:-1]
    hz = np.arange(F) * sr / n_fft
    gap = np.abs(hz[:, None] - pts[None, :]).min() / (sr / n_fft)
    assert gap > 1e-3


def test_structure_invariants():
    for sr, n_fft, nb in [(44100, 2048, 60), (44100, 256, 8)]:
        t = mel.band_tables(sr, n_fft, nb, 2)
        assert t.counts.min() >= 1 and t.counts.max() <= 2
        for b in t.bins:                      # contiguous, ascending
            assert np.all(np.diff(b) == 1)
        assert t.bins[0][0] == 0 and t.bins[-1][-1] == n_fft // 2
        for b, p in zip(t.bins, t.pairs):     # stereo interleave: bin-major, channel-minor
            assert p.tolist() == [k * 2 + s for k in b.tolist() for s in range(2)]


def test_tiny_config_band_bins():
    """The 8-band, n_fft 256 core: derived counts (no printed table exists for it)."""
    t = mel.band_tables(44100, 256, 8, 2)
    assert [len(b) for b in t.bins] == [6, 6, 7, 12, 20, 31, 48, 77]
    assert t.total_width == 828


def test_slaney_scale_closed_forms():
    assert mel.hz_to_mel(1000.0) == pytest.approx(15.0, abs=1e-12)
    assert mel.hz_to_mel(600.0) == pytest.approx(9.0, abs=1e-12)           # 3 mels per 200 Hz
    assert mel.hz_to_mel(6400.0) == pytest.approx(15.0 + 27.0, abs=1e-12)  # 27 mels per factor 6.4
    f = np.array([0.0, 123.0, 999.0, 1000.0, 5000.0, 22050.0])
    assert np.allclose(mel.mel_to_hz(mel.hz_to_mel(f)), f, rtol=1e-13, atol=1e-10)


def test_frames_of_an_8s_chunk():
    assert mel.stft_frames(352800, 441) == 801
