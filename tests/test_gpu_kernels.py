"""Kernel-level checks through the library's test surface (mbr_k_*), against numpy."""
import numpy as np
import pytest

from axial_band_split_amd import binding, synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _dev(a: np.ndarray, dtype: int):
    s = synth.storage_bytes(a, dtype)
    return torch.from_numpy(s.view(np.int16) if s.dtype == np.uint16 else s).cuda()


def _variants() -> int:
    """The 16-bit GEMM's tile configurations (the fp32 GEMM has one)."""
    try:
        return binding.mbr_k_gemm_variants()
    except Exception:      # library not built: collection still works, the tests then fail loudly
        return 1


def _gemm_cases():
    out = []
    for dtype in (synth.F16, synth.BF16, synth.F32):
        for variant in (range(_variants()) if dtype != synth.F32 else [0]):
            for M, N, K in [(1000, 384, 320), (257, 128, 64), (64, 192, 96)]:
                if dtype == synth.F32 and K % 16:
                    continue
                out.append((dtype, variant, M, N, K))
    return out


@pytest.mark.parametrize("dtype,variant,M,N,K", _gemm_cases())
def test_gemm_matches_numpy(dtype, variant, M, N, K):
    print(f"[gemm] dtype={synth.DTYPE_NAMES[dtype]} variant={variant} M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M + N + K + variant)
    a = synth.round_to_dtype(rng.standard_normal((M, K)), dtype)
    b = synth.round_to_dtype(rng.standard_normal((N, K)), dtype)
    bias = rng.standard_normal(N).astype(np.float32)
    A, B = _dev(a, dtype), _dev(b, dtype)
    bd = torch.from_numpy(bias).cuda()
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    binding.mbr_k_gemm(dtype, A.data_ptr(), B.data_ptr(), bd.data_ptr(), C.data_ptr(), M, N, K, variant)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    want = a @ b.T + bias.astype(np.float64)
    err = np.abs(got - want).max() / np.abs(want).max()
    assert np.isfinite(got).all() and err < 1e-5, err


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("variant", range(_variants()))
def test_gemm_16bit_output_matches_numpy(dtype, variant):
    M, N, K = 777, 256, 416
    print(f"[gemm16] dtype={synth.DTYPE_NAMES[dtype]} variant={variant}", flush=True)
    rng = np.random.default_rng(variant + 100)
    a = synth.round_to_dtype(rng.standard_normal((M, K)), dtype)
    b = synth.round_to_dtype(rng.standard_normal((N, K)), dtype)
    bias = rng.standard_normal(N).astype(np.float32)
    A, B = _dev(a, dtype), _dev(b, dtype)
    bd = torch.from_numpy(bias).cuda()
    C = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    binding.mbr_k_gemm(dtype, A.data_ptr(), B.data_ptr(), bd.data_ptr(), C.data_ptr(), M, N, K, variant, out16=True)
    torch.cuda.synchronize()
    raw = C.cpu().numpy()
    got = raw.view(np.float16).astype(np.float64) if dtype == synth.F16 else synth.bf16_bits_to_f64(raw.view(np.uint16))
    want = a @ b.T + bias.astype(np.float64)
    # one rounding of the fp32 result to the 16-bit type
    ulp = 2.0 ** -10 if dtype == synth.F16 else 2.0 ** -7
    assert np.all(np.abs(got - want) <= ulp * np.abs(want) + 1e-3 * np.abs(want).max())


def test_device_gelu_within_the_erf_error_bound():
    """The feed-forward GELU uses A&S 7.1.26 for erf (|error| <= 1.5e-7): compare with math.erf."""
    import math
    xs = np.concatenate([np.linspace(-12, 12, 200001), [0.0, -0.0, 1e-30, -1e-30, 40.0, -40.0]]).astype(np.float32)
    xd = torch.from_numpy(xs).cuda()
    yd = torch.empty_like(xd)
    binding.mbr_k_gelu(xd.data_ptr(), yd.data_ptr(), xs.size)
    torch.cuda.synchronize()
    got = yd.cpu().numpy().astype(np.float64)
    x64 = xs.astype(np.float64)
    want = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x64])
    # erf error: 1.5e-7 from the formula plus single-precision evaluation (reciprocal, exponential
    # and FMA chain, a few ulp of 1.0): 4e-7; GELU multiplies it by x/2, plus rounding of the result
    erf_err = 1.5e-7 + 4 * 2.0 ** -23
    bound = 0.5 * np.abs(x64) * erf_err + 4 * np.spacing(np.abs(want).astype(np.float32)).astype(np.float64) + 1e-37
    assert np.all(np.abs(got - want) <= bound), np.max(np.abs(got - want) / bound)
