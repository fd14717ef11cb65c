"""The steps around the core on the GPU (STFT, masked inverse STFT, chunked separation) against the
oracle's (oracle/pipeline.py), through the C ABI."""
import numpy as np
import pytest

from axial_band_split_amd import binding, synth
from oracle import model as M
from oracle import pipeline as P

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


@pytest.mark.parametrize("n_fft,hop,L", [(2048, 441, 44100 * 2 + 123), (256, 64, 3001), (16, 4, 37)])
def test_stft_matches_oracle(n_fft, hop, L):
    say(f"[stft] n_fft={n_fft} hop={hop} L={L}")
    x = np.random.default_rng(0).standard_normal((2, L)).astype(np.float32)
    got = binding.stft(torch.from_numpy(x).cuda(), n_fft, hop).cpu().numpy()
    want = P.to_core_input(P.stft(x.astype(np.float64), n_fft, hop))
    err = rel_l2(got, want)
    say(f"[stft] rel L2 = {err:.2e}")
    assert got.shape == want.shape and err < 1e-5


@pytest.mark.parametrize("stems", [1, 2])
def test_masked_istft_matches_oracle(stems):
    n_fft, hop, L = 2048, 441, 44100 + 77
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, L))
    z = P.stft(x, n_fft, hop)
    spec = P.to_core_input(z).astype(np.float32)
    masks = rng.uniform(-1, 1, (stems,) + spec.shape[1:]).astype(np.float32)
    got = binding.istft_masked(torch.from_numpy(spec).cuda(), torch.from_numpy(masks).cuda(), 2, L, n_fft, hop)
    got = got.cpu().numpy()
    zz = spec[0, ..., 0].astype(np.float64) + 1j * spec[0, ..., 1]
    zz = np.transpose(zz.reshape(n_fft // 2 + 1, 2, -1), (1, 0, 2))
    y = P.apply_masks(zz, masks.astype(np.float64))
    want = np.stack([P.istft(y[s], n_fft, hop, L) for s in range(stems)])
    err = rel_l2(got, want)
    say(f"[istft] stems {stems}: rel L2 = {err:.2e}")
    assert err < 1e-5


def _unit_mask_weights(w, cfg):
    """Weights whose mask head gives 1 + 0i everywhere: last layer zero, value bias 2 on the real
    features (2 sigmoid(0) = 1), 0 on the imaginary ones, gate bias 0."""
    ws = synth.draw_weights(binding.inventory(cfg), w.dtype, seed=0)
    oc = M.CoreConfig(w.sample_rate, w.n_fft, w.audio_channels, w.num_bands, w.dim, w.depth, w.heads, w.dim_head,
                      w.ff_mult, w.mask_hidden_mult, w.mask_depth, w.num_stems)
    for idx, (name, shape, _) in enumerate(M.inventory(oc)):
        if name.startswith("stem") and name.endswith(f"mlp{w.mask_depth}.weight"):
            ws[idx] = np.zeros(shape)
        if name.startswith("stem") and name.endswith(f"mlp{w.mask_depth}.bias"):
            W = shape[0] // 2
            b = np.zeros(2 * W)
            b[0:W:2] = 2.0
            ws[idx] = b
    return ws


def test_separation_with_unit_masks_returns_the_track_full_size():
    """The vocals architecture at 801 frames (8 s chunks), fp16, max_batch 4, on 40 s of stereo noise:
    with masks of exactly 1 + 0i the separation is the identity up to fp32 STFT rounding."""
    w = synth.WORKLOADS["chunk11s_fp16"].replace(frames=801, batch=4)
    cfg = binding.config(w)
    core = binding.Core(cfg, _unit_mask_weights(w, cfg))
    L = 44100 * 40 + 1234
    x = np.random.default_rng(3).standard_normal((2, L)).astype(np.float32)
    say(f"[separate] unit masks, {L} samples")
    y = core.separate(torch.from_numpy(x).cuda(), 441).cpu().numpy()
    core.close()
    err = rel_l2(y[0], x)
    say(f"[separate] rel L2 = {err:.2e}")
    assert y.shape == (1, 2, L) and err < 1e-5


@pytest.mark.parametrize("L,stems", [(7000, 1), (2500, 2), (9333, 1)])
def test_separation_matches_oracle_tiny_core(L, stems):
    """The tiny fp32 core (n_fft 256, 8 bands) with 33 frames: 2048-sample chunks, hop 64, two chunks
    per core call; full, reflected and zero-padded tails."""
    w = synth.WORKLOADS["tiny_fp32"].replace(frames=33, batch=2, num_stems=stems)
    cfg = binding.config(w)
    ws = synth.draw_weights(binding.inventory(cfg), w.dtype, seed=0, std=0.1)
    oc = M.CoreConfig(w.sample_rate, w.n_fft, w.audio_channels, w.num_bands, w.dim, w.depth, w.heads, w.dim_head,
                      w.ff_mult, w.mask_hidden_mult, w.mask_depth, w.num_stems)
    x = np.random.default_rng(4).standard_normal((2, L)).astype(np.float32)
    say(f"[separate] tiny core, L={L}, stems {stems}")
    core = binding.Core(cfg, ws)
    got = core.separate(torch.from_numpy(x).cuda(), 64).cpu().numpy()
    core.close()

    def oracle_core(spec):
        m = M.forward(spec, oc, ws)
        return m if stems == 1 else m[0]

    want = P.separate(x.astype(np.float64), oracle_core, 256, 64, 2048, stems)
    err = rel_l2(got, want)
    say(f"[separate] rel L2 = {err:.2e}")
    assert got.shape == want.shape and err < 1e-4


def test_separation_half_precision_vocals_core_matches_oracle():
    """The vocals architecture (60 bands, D 384, depth 6) in fp16 at 97 frames (42336-sample chunks):
    a 100000-sample synthetic track gives three chunks, the last one with a reflected tail, two per
    core call.  The waveforms against the oracle's separation with its fp64 core on the same weights."""
    w = synth.WORKLOADS["t256_fp16"].replace(frames=97, batch=2)
    cfg = binding.config(w)
    ws = synth.draw_weights(binding.inventory(cfg), w.dtype, seed=w.weight_seed)
    oc = M.CoreConfig(w.sample_rate, w.n_fft, w.audio_channels, w.num_bands, w.dim, w.depth, w.heads, w.dim_head,
                      w.ff_mult, w.mask_hidden_mult, w.mask_depth, w.num_stems)
    x = synth.draw_wave(2, 100000, seed=7)
    say("[separate] vocals fp16, 97 frames, 100000 samples")
    core = binding.Core(cfg, ws)
    got = core.separate(torch.from_numpy(x).cuda(), 441).cpu().numpy()
    core.close()
    want = P.separate(x.astype(np.float64), lambda spec: M.forward(spec, oc, ws), 2048, 441, 96 * 441, 1)
    err = rel_l2(got, want)
    say(f"[separate] rel L2 = {err:.2e}")
    assert got.shape == want.shape and err < 2e-2


@pytest.mark.parametrize("L", [2, 100, 1500])
def test_separation_of_tracks_shorter_than_a_chunk(L):
    """Tracks of 2 samples (the shortest accepted), 100 (under two borders: no reflect padding, one
    zero-padded chunk) and 1500 (reflect-padded to 1910: one chunk with a reflected tail, then 67
    samples in a zero-padded one) through the tiny fp32 core (2048-sample chunks, hop 64), against
    the oracle's separation."""
    w = synth.WORKLOADS["tiny_fp32"].replace(frames=33, batch=2)
    cfg = binding.config(w)
    ws = synth.draw_weights(binding.inventory(cfg), w.dtype, seed=0, std=0.1)
    oc = M.CoreConfig(w.sample_rate, w.n_fft, w.audio_channels, w.num_bands, w.dim, w.depth, w.heads, w.dim_head,
                      w.ff_mult, w.mask_hidden_mult, w.mask_depth, w.num_stems)
    x = np.random.default_rng(5).standard_normal((2, L)).astype(np.float32)
    say(f"[separate] tiny core, short track L={L}")
    core = binding.Core(cfg, ws)
    got = core.separate(torch.from_numpy(x).cuda(), 64).cpu().numpy()
    core.close()
    want = P.separate(x.astype(np.float64), lambda spec: M.forward(spec, oc, ws), 256, 64, 2048, 1)
    err = rel_l2(got, want)
    say(f"[separate] rel L2 = {err:.2e}")
    assert got.shape == want.shape == (1, 2, L) and err < 1e-4


def test_separation_refuses_a_one_sample_track():
    w = synth.WORKLOADS["tiny_fp32"].replace(frames=33, batch=1)
    cfg = binding.config(w)
    core = binding.Core(cfg, synth.draw_weights(binding.inventory(cfg), w.dtype, seed=0))
    x = torch.zeros((2, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.MbrError):
        core.separate(x, 64)
    core.close()


@pytest.mark.parametrize("L,stride", [(7000, 1024), (9333, 1024), (2500, 700)])
def test_strided_separation_matches_oracle_tiny_core(L, stride):
    """The separation with a chosen stride: half a chunk ([P4] "Graph": segments every half chunk,
    the border as large), and an odd stride; tiny fp32 core, 2048-sample chunks, two per core call."""
    w = synth.WORKLOADS["tiny_fp32"].replace(frames=33, batch=2)
    cfg = binding.config(w)
    ws = synth.draw_weights(binding.inventory(cfg), w.dtype, seed=0, std=0.1)
    oc = M.CoreConfig(w.sample_rate, w.n_fft, w.audio_channels, w.num_bands, w.dim, w.depth, w.heads, w.dim_head,
                      w.ff_mult, w.mask_hidden_mult, w.mask_depth, w.num_stems)
    x = np.random.default_rng(8).standard_normal((2, L)).astype(np.float32)
    say(f"[separate] tiny core, L={L}, stride {stride}")
    core = binding.Core(cfg, ws)
    got = core.separate(torch.from_numpy(x).cuda(), 64, stride=stride).cpu().numpy()
    core.close()
    want = P.separate(x.astype(np.float64), lambda spec: M.forward(spec, oc, ws), 256, 64, 2048, 1, stride=stride)
    err = rel_l2(got, want)
    say(f"[separate] rel L2 = {err:.2e}")
    assert got.shape == want.shape and err < 1e-4


def test_separation_refuses_a_stride_past_the_fades():
    """A stride over chunk - chunk/10 (2048-sample chunks: 1844) would leave samples without a chunk
    of full weight: 1845 is MBR_E_ARG before anything is launched; 1844 is accepted."""
    w = synth.WORKLOADS["tiny_fp32"].replace(frames=33, batch=1)
    cfg = binding.config(w)
    core = binding.Core(cfg, synth.draw_weights(binding.inventory(cfg), w.dtype, seed=0))
    assert binding.mbr_separate_workspace_size_strided(core.handle, 5000, 64, 1844) > 0
    with pytest.raises(binding.MbrError) as e:
        binding.mbr_separate_workspace_size_strided(core.handle, 5000, 64, 1845)
    assert e.value.code == binding.MBR_E_ARG
    core.close()
