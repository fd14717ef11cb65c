"""The allocation-free inverse STFT (mbr_istft_masked_noalloc) against mbr_istft_masked, through the
C ABI: two calls in a row on one GPU, the second smaller, each bitwise equal to the entry point with
a caller workspace; a size past the static buffer is refused before anything is launched."""
import numpy as np
import pytest

from axial_band_split_amd import binding

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)


def _inputs(stems, channels, length, n_fft, hop, seed):
    rng = np.random.default_rng(seed)
    T, F = 1 + length // hop, n_fft // 2 + 1
    spec = rng.standard_normal((1, F * channels, T, 2)).astype(np.float32)
    masks = rng.uniform(-1, 1, (stems, F * channels, T, 2)).astype(np.float32)
    return torch.from_numpy(spec).cuda(), torch.from_numpy(masks).cuda()


def test_noalloc_istft_matches_the_workspace_entry_point_twice():
    n_fft, hop = 2048, 441
    for stems, length, seed in ((2, 44100 * 3 + 17, 0), (1, 20000, 1)):
        say(f"[noalloc] stems={stems} length={length}")
        spec, masks = _inputs(stems, 2, length, n_fft, hop, seed)
        T = spec.shape[2]
        ws = torch.empty(binding.mbr_istft_workspace_size(2, n_fft, T, stems), dtype=torch.uint8, device="cuda")
        want = torch.full((stems, 2, length), float("nan"), device="cuda")
        got = torch.full((stems, 2, length), float("nan"), device="cuda")
        s = torch.cuda.current_stream().cuda_stream
        binding.mbr_istft_masked(spec.data_ptr(), masks.data_ptr(), stems, 2, length, n_fft, hop, ws.data_ptr(),
                                 want.data_ptr(), s)
        binding.mbr_istft_masked_noalloc(spec.data_ptr(), masks.data_ptr(), stems, 2, length, n_fft, hop,
                                         got.data_ptr(), s)
        torch.cuda.synchronize()
        assert torch.isfinite(want).all()
        assert torch.equal(got, want), f"stems={stems} length={length}"


def test_noalloc_istft_refuses_sizes_past_its_buffer():
    n_fft, hop, stems, channels = 2048, 441, 1, 2
    frames = binding.MBR_ISTFT_NOALLOC_MAX_BYTES // (stems * channels * n_fft * 4) + 1
    length = (frames - 1) * hop
    dummy = torch.zeros(4, device="cuda")
    with pytest.raises(binding.MbrError) as e:
        binding.mbr_istft_masked_noalloc(dummy.data_ptr(), dummy.data_ptr(), stems, channels, length, n_fft, hop,
                                         dummy.data_ptr(), 0)
    assert e.value.code == binding.MBR_E_ARG and "static buffer" in binding.mbr_last_error()
