"""Error behaviour of libmbr_core.so's entry points that the host decides (no GPU needed): each case
below is refused by the library's argument checks before any HIP call, so the placeholder
pointers are never dereferenced; and with no GPU visible, creating a core fails with a device
error instead of running anywhere else."""
import numpy as np
import pytest

from axial_band_split_amd import binding, synth

E_ARG, E_HIP, E_DEVICE = -1, -4, -3
F32, F16, BF16 = synth.F32, synth.F16, synth.BF16

_buf = np.zeros(64, dtype=np.float32)     # a valid host address to stand in for operands
P = _buf.ctypes.data


def _gemm(**kw):
    a = dict(dtype=F16, a_ptr=P, b_ptr=P, bias_ptr=0, c_ptr=P, M=64, N=64, K=64, variant=0, out16=False)
    a.update(kw)
    return lambda: binding.mbr_k_gemm(**a)


def _attn(**kw):
    a = dict(dtype=F16, q_ptr=P, k_ptr=P, vt_ptr=P, gates_ptr=0, o_ptr=P, seqs=1, heads=1, n=100, npad=128,
             dqk=64, dv=64, scale=0.125)
    a.update(kw)
    return lambda: binding.mbr_attention(**a)


CASES = {
    "gemm: NULL operand": (_gemm(a_ptr=0), "NULL"),
    "gemm: N not a multiple of 64": (_gemm(N=100), "N % 64"),
    "gemm: K not a multiple of the 16-bit K step": (_gemm(K=48), "K step"),
    "gemm: fp32 K not a multiple of 16": (_gemm(dtype=F32, K=40), "K step"),
    "gemm: M = 0": (_gemm(M=0), "N % 64"),
    "gemm: unknown tile variant": (_gemm(variant=99), "variant"),
    "gemm: unknown dtype": (_gemm(dtype=7), "dtype"),
    "gemm: 16-bit output from fp32": (_gemm(dtype=F32, out16=True), "16-bit output"),
    "attention: NULL operand": (_attn(o_ptr=0), "NULL"),
    "attention: fp32": (_attn(dtype=F32), "dtype"),
    "attention: npad not a multiple of 128": (_attn(npad=192), "multiple of 128"),
    "attention: n above npad": (_attn(n=129), "npad"),
    "attention: n = 0": (_attn(n=0), "npad"),
    "attention: v wider than q/k": (_attn(dqk=64, dv=128), "(dqk, dv)"),
    "attention: unsupported width pair": (_attn(dqk=128, dv=128), "(dqk, dv)"),
    "attention: zero scale": (_attn(scale=0.0), "scale"),
    "attention: NaN scale": (_attn(scale=float("nan")), "scale"),
    "attention: infinite scale": (_attn(scale=float("inf")), "scale"),
    "stft: NULL wave": (lambda: binding.mbr_stft(0, 2, 44100, 2048, 441, P), "NULL"),
    "stft: n_fft not a power of two": (lambda: binding.mbr_stft(P, 2, 44100, 2000, 441, P), "power of two"),
    "stft: hop above n_fft / 2": (lambda: binding.mbr_stft(P, 2, 44100, 2048, 1025, P), "hop"),
    "stft: one sample": (lambda: binding.mbr_stft(P, 2, 1, 2048, 441, P), "length"),
    "istft: NULL workspace": (lambda: binding.mbr_istft_masked(P, P, 1, 2, 44100, 2048, 441, 0, P), "NULL"),
    "istft: no stems": (lambda: binding.mbr_istft_masked(P, P, 0, 2, 44100, 2048, 441, P, P), "bad sizes"),
    "istft workspace: n_fft not supported": (lambda: binding.mbr_istft_workspace_size(2, 1000, 101, 1), "bad sizes"),
    "istft workspace: no frames": (lambda: binding.mbr_istft_workspace_size(2, 2048, 0, 1), "bad sizes"),
    # 4 stems x 2 channels x 3001 frames x 2048 x 4 bytes = 196.7 MB, over the 64 MiB static buffer
    "istft without allocation: over the static buffer": (
        lambda: binding.mbr_istft_masked_noalloc(P, P, 4, 2, 441 * 3000, 2048, 441, P), "exceeds the static buffer"),
    "istft without allocation: NULL output": (
        lambda: binding.mbr_istft_masked_noalloc(P, P, 1, 2, 44100, 2048, 441, 0), "NULL"),
    "forward: NULL core": (lambda: binding.mbr_core_forward(None, P, P, 1), "NULL"),
    "debug size: NULL core": (lambda: binding.mbr_core_debug_size(None, 1, 0), "bad core"),
    "separate workspace: NULL core": (lambda: binding.mbr_separate_workspace_size(None, 44100, 441), "NULL core"),
    "separate: NULL core": (lambda: binding.mbr_separate(None, P, 44100, 441, P, P), "NULL"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_bad_arguments_are_refused(case):
    call, words = CASES[case]
    with pytest.raises(binding.MbrError) as e:
        call()
    assert e.value.code == E_ARG
    assert words in binding.mbr_last_error()


def test_istft_workspace_size_is_the_frame_buffer():
    # stems x channels x frames x n_fft fp32 values: the windowed frames before overlap-add
    assert binding.mbr_istft_workspace_size(2, 2048, 101, 4) == 4 * 2 * 101 * 2048 * 4
    assert binding.mbr_istft_workspace_size(1, 16, 1, 1) == 16 * 4


def test_device_bytes_of_no_core_is_zero():
    assert binding.mbr_core_device_bytes(None) == 0


def test_core_creation_without_a_gpu_fails_loudly():
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: core creation would go ahead (the GPU tests cover it)")
    cfg = binding.config(synth.WORKLOADS["tiny_fp32"])
    n = binding.mbr_core_weight_count(cfg)
    with pytest.raises(binding.MbrError) as e:
        binding.mbr_core_create(cfg, [P] * n)
    assert e.value.code in (E_HIP, E_DEVICE)


def test_config_errors_come_before_the_device_check():
    """A bad configuration is reported as such on any host, GPU or not."""
    cfg = binding.config(synth.WORKLOADS["tiny_fp32"], n_fft=32, num_bands=40)
    n = 1
    with pytest.raises(binding.MbrError) as e:
        binding.mbr_core_create(cfg, [P] * n)
    assert e.value.code == -2
