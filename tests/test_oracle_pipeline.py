"""Pins of the oracle's STFT / iSTFT / chunked overlap-add (oracle/pipeline.py), CPU only."""
import numpy as np
import pytest

from oracle import pipeline as P


def test_stft_equals_the_direct_transform():
    """A centred, Hann-windowed, reflect-padded DFT written out term by term."""
    rng = np.random.default_rng(0)
    n_fft, hop, L = 16, 4, 37
    x = rng.standard_normal((2, L))
    got = P.stft(x, n_fft, hop)
    T = 1 + L // hop
    assert got.shape == (2, n_fft // 2 + 1, T)
    want = np.zeros_like(got)
    for c in range(2):
        for t in range(T):
            for k in range(n_fft // 2 + 1):
                acc = 0.0
                for n in range(n_fft):
                    i = t * hop + n - n_fft // 2
                    while i < 0 or i >= L:                       # mirror about the end samples
                        i = -i if i < 0 else 2 * (L - 1) - i
                    wn = 0.5 - 0.5 * np.cos(2 * np.pi * n / n_fft)
                    acc += wn * x[c, i] * np.exp(-2j * np.pi * k * n / n_fft)
                want[c, k, t] = acc
    assert np.allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n_fft,hop,L", [(2048, 441, 44100), (256, 64, 3001), (16, 4, 37)])
def test_istft_inverts_stft(n_fft, hop, L):
    """Hann window, hop <= n_fft / 2: the windowed overlap-add over the summed squared window
    gives the signal back exactly."""
    x = np.random.default_rng(1).standard_normal((2, L))
    y = P.istft(P.stft(x, n_fft, hop), n_fft, hop, L)
    assert np.allclose(y, x, rtol=0, atol=1e-11)


def test_chunk_arithmetic_of_the_pages():
    """8 s at 44.1 kHz: chunk 352800, stride 317520 (7.2 s), fade and border 35280 (0.8 s)."""
    chunk = 44100 * 8
    Lp, pad, plan = P.chunk_plan(60 * 44100, chunk)
    assert pad == 35280 and Lp == 60 * 44100 + 2 * 35280
    assert [o for o, _, _ in plan][:3] == [0, 317520, 635040]
    assert P.fade_window(chunk, False, False)[:35280].tolist() == np.linspace(0, 1, 35280).tolist()
    # a short track is not padded
    assert P.chunk_plan(50000, chunk)[1] == 0


def test_fades_are_a_partition_of_unity():
    chunk = 1000
    Lp, pad, plan = P.chunk_plan(5300, chunk)
    counter = np.zeros(Lp)
    stride = int(chunk * 0.9)
    for ci, (off, n, _) in enumerate(plan):
        counter[off:off + n] += P.fade_window(chunk, ci == 0, off + stride >= Lp)[:n]
    assert np.allclose(counter, 1.0, rtol=0, atol=1e-15)


@pytest.mark.parametrize("L", [2500, 7000, 9333])
def test_separation_with_unit_masks_returns_the_track(L):
    """Masks 1 + 0i for every stem: STFT, iSTFT and the faded overlap-add must give the track back
    (zero- and reflect-padded tails included)."""
    n_fft, hop, chunk = 256, 64, 2048
    wave = np.random.default_rng(2).standard_normal((2, L))

    def unit_core(spec):
        m = np.zeros((2,) + spec.shape[1:])
        m[..., 0] = 1.0
        return m

    modes = {mode for _, _, mode in P.chunk_plan(L, chunk)[2]}
    out = P.separate(wave, unit_core, n_fft, hop, chunk, stems=2)
    assert out.shape == (2, 2, L)
    assert np.allclose(out[0], wave, rtol=0, atol=1e-10) and np.allclose(out[1], wave, rtol=0, atol=1e-10)
    assert modes <= {"full", "reflect", "zero"}


def test_chunk_tails_cover_both_padding_modes():
    """The lengths of the unit-mask test reach both tail modes (7000: a reflected and a zero-padded
    tail; 2500: a reflected one)."""
    assert {m for _, _, m in P.chunk_plan(7000, 2048)[2]} == {"full", "reflect", "zero"}
    assert {m for _, _, m in P.chunk_plan(2500, 2048)[2]} == {"full", "reflect"}


def test_core_input_layout_element_by_element():
    """stft_repr [1, F*S, T, 2] holds channel s of bin f at pair f*S + s, real part first ([P1] "The
    forward chain": the stereo channels merged into the frequency axis, bin-major)."""
    rng = np.random.default_rng(3)
    S, F, T = 2, 5, 4
    z = rng.standard_normal((S, F, T)) + 1j * rng.standard_normal((S, F, T))
    x = P.to_core_input(z)
    assert x.shape == (1, F * S, T, 2)
    for s in range(S):
        for f in range(F):
            for t in range(T):
                assert x[0, f * S + s, t, 0] == z[s, f, t].real
                assert x[0, f * S + s, t, 1] == z[s, f, t].imag


def test_mask_product_with_non_unit_masks():
    """Masks in the core's layout multiply the STFT as complex numbers, each channel by its own
    pair: real constants a (left) and b (right) give a z_L and b z_R, a different pair per stem;
    0 + 1i applied twice gives -z; one element checked against the complex product written out."""
    rng = np.random.default_rng(4)
    S, F, T = 2, 6, 3
    z = rng.standard_normal((S, F, T)) + 1j * rng.standard_normal((S, F, T))
    m = np.zeros((2, F * S, T, 2))
    m[0, 0::2, :, 0], m[0, 1::2, :, 0] = 0.25, -3.0        # stem 0: a = 0.25 on the left, b = -3 on the right
    m[1, 0::2, :, 0], m[1, 1::2, :, 0] = 2.0, 0.5          # stem 1: a = 2, b = 0.5
    y = P.apply_masks(z, m)
    assert y.shape == (2, S, F, T)
    assert np.array_equal(y[0, 0], 0.25 * z[0]) and np.array_equal(y[0, 1], -3.0 * z[1])
    assert np.array_equal(y[1, 0], 2.0 * z[0]) and np.array_equal(y[1, 1], 0.5 * z[1])
    i = np.zeros((1, F * S, T, 2))
    i[..., 1] = 1.0
    twice = P.apply_masks(P.apply_masks(z, i)[0], i)[0]
    assert np.allclose(twice, -z, rtol=0, atol=1e-15)
    g = rng.standard_normal((1, F * S, T, 2))
    y = P.apply_masks(z, g)
    s, f, t = 1, 4, 2
    mr, mi = g[0, f * S + s, t]
    zr, zi = z[s, f, t].real, z[s, f, t].imag
    assert y[0, s, f, t] == complex(zr * mr - zi * mi, zr * mi + zi * mr)


def test_segments_every_half_chunk():
    """[P4] "Graph": 8 s segments every 4 s faded over 0.8 s, the input reflected out at the ends:
    stride 176400, border (reflect pad) 176400, fades of 35280 samples."""
    chunk = 44100 * 8
    Lp, pad, plan = P.chunk_plan(60 * 44100, chunk, chunk // 2)
    assert pad == 176400 and Lp == 60 * 44100 + 2 * 176400
    assert [o for o, _, _ in plan][:4] == [0, 176400, 352800, 529200]
    assert len(plan) == -(-Lp // 176400)


@pytest.mark.parametrize("L", [2500, 7000, 9333])
def test_half_chunk_separation_with_unit_masks_returns_the_track(L):
    n_fft, hop, chunk = 256, 64, 2048
    wave = np.random.default_rng(6).standard_normal((2, L))

    def unit_core(spec):
        m = np.zeros((1,) + spec.shape[1:])
        m[..., 0] = 1.0
        return m

    out = P.separate(wave, unit_core, n_fft, hop, chunk, stems=1, stride=chunk // 2)
    assert out.shape == (1, 2, L)
    assert np.allclose(out[0], wave, rtol=0, atol=1e-10)


@pytest.mark.parametrize("stride", [None, 1024])
def test_separation_with_constant_masks_scales_each_stem_and_channel(stride):
    """Real masks c[stem, channel] (pair p = f * S + s): the iSTFT is linear and the fades sum to
    one, so stem k's channel s comes back as c[k, s] times the track's channel s; masks that were
    ignored, or stems or channels taken in the wrong order, fail this."""
    n_fft, hop, chunk, L = 256, 64, 2048, 7000
    S = 2
    wave = np.random.default_rng(8).standard_normal((S, L))
    c = np.array([[0.25, -1.5], [2.0, 0.5], [-0.75, 3.0]])          # [stems, channels]

    def const_core(spec):
        FS = spec.shape[1]
        m = np.zeros((3,) + spec.shape[1:])
        for k in range(3):
            for s in range(S):
                m[k, s:FS:S, :, 0] = c[k, s]
        return m

    out = P.separate(wave, const_core, n_fft, hop, chunk, stems=3, stride=stride)
    assert out.shape == (3, S, L)
    for k in range(3):
        for s in range(S):
            assert np.allclose(out[k, s], c[k, s] * wave[s], rtol=0, atol=1e-9)
