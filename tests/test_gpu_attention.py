"""The standalone gated attention (mbr_attention) against the oracle's (oracle/attention.py), through
the C ABI: q and k twice as wide as v ([P2] "Evaluation record", "BS PolarFormer..." part "Ported, and
what it actually bought": 62 bands, 8 heads of 64, chunks of 588800 samples at hop 512 = 1151 frames),
and q, k, v of one width."""
import numpy as np
import pytest

from axial_band_split_amd import binding, synth
from oracle import attention as A

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
TOL = 2e-2


def say(*a):
    print(*a, flush=True)


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


def _dev(a, dtype):
    b = synth.storage_bytes(a, dtype)
    return torch.from_numpy(b.view(np.int16) if b.dtype == np.uint16 else b).cuda()


def _from_dev(t, dtype):
    a = t.cpu().numpy()
    if dtype == synth.BF16:
        return synth.bf16_bits_to_f64(a.view(np.uint16))
    return a.astype(np.float64)


def run_case(dtype, seqs, heads, n, dqk, dv, scale, seed, gated=True):
    rng = np.random.default_rng(seed)
    npad = -(-n // 128) * 128
    q = synth.round_to_dtype(rng.standard_normal((seqs, heads, n, dqk)), dtype)
    k = synth.round_to_dtype(rng.standard_normal((seqs, heads, n, dqk)), dtype)
    v = synth.round_to_dtype(rng.standard_normal((seqs, heads, n, dv)), dtype)
    g = rng.uniform(0.05, 1.0, (seqs, n, heads)) if gated else None
    pad = ((0, 0), (0, 0), (0, npad - n), (0, 0))
    qd, kd = _dev(np.pad(q, pad), dtype), _dev(np.pad(k, pad), dtype)
    vtd = _dev(np.ascontiguousarray(np.swapaxes(np.pad(v, pad), -1, -2)), dtype)
    gd = torch.from_numpy(g.astype(np.float32)).cuda() if gated else None
    od = torch.empty((seqs, n, heads * dv), dtype=torch.int16, device="cuda")
    binding.mbr_attention(dtype, qd.data_ptr(), kd.data_ptr(), vtd.data_ptr(), gd.data_ptr() if gated else 0,
                          od.data_ptr(), seqs, heads, n, npad, dqk, dv, scale, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = _from_dev(od if dtype == synth.BF16 else od.view(torch.float16), dtype)
    want = A.gated_attention(q, k, v, scale, g.astype(np.float32).astype(np.float64) if gated else None)
    return got, want


@pytest.mark.parametrize("dtype,seqs,n", [(synth.F16, 62, 1151), (synth.BF16, 62, 1151), (synth.F16, 5, 97)])
def test_narrow_v_attention_matches_oracle(dtype, seqs, n):
    say(f"[attn] q/k 128, v 64, {synth.DTYPE_NAMES[dtype]}, {seqs} sequences x 8 heads, n={n}")
    got, want = run_case(dtype, seqs, 8, n, 128, 64, 128 ** -0.5, seed=n)
    err = rel_l2(got, want)
    per_seq = max(rel_l2(got[s], want[s]) for s in range(seqs))
    say(f"[attn] rel L2 = {err:.2e}, worst sequence {per_seq:.2e}")
    assert np.isfinite(got).all() and err <= TOL and per_seq <= TOL


def test_narrow_v_attention_with_peaked_scores():
    """Scale 1 instead of 1/sqrt(128): scores of standard deviation about 11, so the reference of the
    exponentials moves past its first key tile for many queries; no gates (all 1)."""
    say("[attn] q/k 128, v 64, peaked scores, no gates")
    got, want = run_case(synth.F16, 6, 8, 700, 128, 64, 1.0, seed=11, gated=False)
    err = rel_l2(got, want)
    say(f"[attn] rel L2 = {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("dqk", [64, 32])
def test_equal_width_attention_matches_oracle(dqk):
    got, want = run_case(synth.BF16, 4, 8, 300, dqk, dqk, dqk ** -0.5, seed=dqk)
    err = rel_l2(got, want)
    say(f"[attn] q/k/v {dqk}: rel L2 = {err:.2e}")
    assert err <= TOL


def test_attention_refuses_bad_shapes():
    x = torch.zeros(1 << 16, dtype=torch.int16, device="cuda")
    p = x.data_ptr()
    for args in [(synth.F16, 1, 8, 100, 100, 128, 64, 0.1),      # npad not a multiple of 128
                 (synth.F16, 1, 8, 200, 128, 128, 64, 0.1),      # n > npad
                 (synth.F16, 1, 8, 100, 128, 64, 128, 0.1),      # v wider than q
                 (synth.F32, 1, 8, 100, 128, 128, 64, 0.1),      # fp32 operands
                 (synth.F16, 1, 8, 100, 128, 128, 64, 0.0)]:     # scale 0
        dt, s, h, n, npad, dqk, dv, sc = args
        with pytest.raises(binding.MbrError) as e:
            binding.mbr_attention(dt, p, p, p, 0, p, s, h, n, npad, dqk, dv, sc, 0)
        assert e.value.code == binding.MBR_E_ARG
