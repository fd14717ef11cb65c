"""The seeded input generators that serve both the oracle and the library: rounding to the storage
types, the storage encoding, and the stated distributions of the synthetic weights, spectra and
tracks (no GPU needed)."""
import numpy as np
import pytest

from axial_band_split_amd import synth

torch = pytest.importorskip("torch")


def _values(n=200000, seed=0):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(n) * np.exp2(rng.integers(-140, 120, n))      # normal and subnormal range
    special = [0.0, -0.0, np.inf, -np.inf, 1.0, -1.0, 65504.0, 3.3895313892515355e38, 1e-45, -1e-45]
    return np.concatenate([v, special]).astype(np.float32)


def test_bf16_rounding_matches_torch_bit_for_bit():
    """fp32 -> bf16 round to nearest, ties to even, against torch's conversion (finite, infinite,
    subnormal and overflowing values)."""
    a = _values()
    ours = synth.f64_to_bf16_bits(a.astype(np.float64))
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_ties_round_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even is 1; 1 + 3 * 2^-8 goes up to 1 + 2^-6
    got = synth.round_to_dtype(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20]),
                               synth.BF16)
    assert got.tolist() == [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7]


def test_bf16_nan_stays_nan():
    bits = synth.f64_to_bf16_bits(np.array([np.nan, -np.nan]))
    assert np.isnan(synth.bf16_bits_to_f64(bits)).all()


@pytest.mark.parametrize("dtype", [synth.F32, synth.F16, synth.BF16])
def test_storage_encodes_exactly_the_rounded_values(dtype):
    """What the library is handed decodes to the same numbers the oracle computes with."""
    rng = np.random.default_rng(1)
    a = rng.standard_normal(50000) * 0.05
    r = synth.round_to_dtype(a, dtype)
    s = synth.storage_bytes(r, dtype)
    back = synth.bf16_bits_to_f64(s) if dtype == synth.BF16 else s.astype(np.float64)
    assert np.array_equal(back, r)
    assert np.array_equal(synth.round_to_dtype(r, dtype), r)                # rounding is idempotent
    ulp = {synth.F32: 2.0 ** -24, synth.F16: 2.0 ** -11, synth.BF16: 2.0 ** -8}[dtype]
    small = np.abs(a) < 6.2e-5 if dtype == synth.F16 else np.zeros(a.shape, bool)   # f16 subnormals
    assert np.all(np.abs(r - a)[~small] <= ulp * np.abs(a)[~small])


def test_weights_are_seeded_and_follow_their_kinds():
    inv = [("w", (256, 512), synth.KIND_MATRIX), ("g", (4096,), synth.KIND_GAMMA)]
    w1 = synth.draw_weights(inv, synth.F32, seed=3)
    w2 = synth.draw_weights(inv, synth.F32, seed=3)
    w3 = synth.draw_weights(inv, synth.F32, seed=4)
    assert all(np.array_equal(a, b) for a, b in zip(w1, w2))
    assert not np.array_equal(w1[0], w3[0])
    assert abs(w1[0].mean()) < 1e-3 and w1[0].std() == pytest.approx(0.02, rel=0.02)
    assert w1[1].mean() == pytest.approx(1.0, abs=2e-3) and w1[1].std() == pytest.approx(0.02, rel=0.05)


def test_normal_spectrum_statistics():
    w = synth.WORKLOADS["tiny_fp32"].replace(input_kind="normal", frames=64, batch=2)
    x = synth.draw_input(w)
    assert x.shape == (2, w.freqs * w.audio_channels, 64, 2) and x.dtype == np.float32
    assert abs(x.mean()) < 0.02 and x.std() == pytest.approx(1.0, rel=0.02)
    assert np.array_equal(x, synth.draw_input(w))
    assert not np.array_equal(x, synth.draw_input(w, seed=w.input_seed + 1))


def test_one_over_f_spectrum_statistics():
    """Magnitude |Laplace(0, 1)| / max(f, 1), phase uniform: |x| * max(f, 1) has mean 1 and the
    phase's cosine mean 0, at every bin and channel (pair p = f * S + s)."""
    w = synth.WORKLOADS["tiny_fp32"].replace(input_kind="one_over_f", frames=256, batch=2)
    x = synth.draw_input(w).astype(np.float64)
    F, S = w.freqs, w.audio_channels
    mag = np.hypot(x[..., 0], x[..., 1]).reshape(2, F, S, 256)
    scaled = mag * np.maximum(np.arange(F), 1.0)[None, :, None, None]
    assert scaled.mean() == pytest.approx(1.0, rel=0.02)
    per_bin = scaled.mean(axis=(0, 2, 3))
    assert np.all(np.abs(per_bin - 1.0) < 0.25)              # 1024 draws per bin
    phase = np.arctan2(x[..., 1], x[..., 0])
    assert abs(np.cos(phase).mean()) < 0.02 and abs(np.sin(phase).mean()) < 0.02


def test_track_rms_and_channel_correlation():
    """A common part plus half as much private noise per channel: correlation 1 / (1 + 0.25)."""
    x = synth.draw_wave(2, 441000, seed=5).astype(np.float64)
    assert np.sqrt(np.mean(x * x)) == pytest.approx(0.1, rel=1e-5)
    c = np.corrcoef(x[0], x[1])[0, 1]
    assert c == pytest.approx(0.8, abs=0.03)
    assert np.array_equal(x, synth.draw_wave(2, 441000, seed=5))
