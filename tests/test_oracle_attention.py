"""Pins of the oracle's gated attention with v narrower than q and k (oracle/attention.py), CPU only."""
import math

import numpy as np
import pytest

from oracle import attention as A


def _brute(q, k, v, scale, gates):
    """Scalar loops: every score, the softmax with the plain sum of exponentials (no max shift)."""
    S, H, n, dqk = q.shape
    dv = v.shape[-1]
    o = np.zeros((S, n, H * dv))
    for s in range(S):
        for h in range(H):
            for t in range(n):
                e = [math.exp(scale * sum(q[s, h, t, d] * k[s, h, j, d] for d in range(dqk))) for j in range(n)]
                z = sum(e)
                for d in range(dv):
                    o[s, t, h * dv + d] = gates[s, t, h] * sum(e[j] * v[s, h, j, d] for j in range(n)) / z
    return o


@pytest.mark.parametrize("dqk,dv", [(8, 4), (6, 6), (4, 2)])
def test_matches_brute_force(dqk, dv):
    rng = np.random.default_rng(0)
    S, H, n = 2, 3, 5
    q, k = rng.standard_normal((S, H, n, dqk)), rng.standard_normal((S, H, n, dqk))
    v, g = rng.standard_normal((S, H, n, dv)), rng.uniform(0.1, 1.0, (S, n, H))
    got = A.gated_attention(q, k, v, dqk ** -0.5, g)
    assert np.allclose(got, _brute(q, k, v, dqk ** -0.5, g), rtol=0, atol=1e-12)


def test_rows_sum_to_one_and_one_key_gives_v():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((2, 2, 7, 8)), rng.standard_normal((2, 2, 7, 8))
    ones = np.ones((2, 2, 7, 4))
    assert np.allclose(A.gated_attention(q, k, ones, 0.7), 1.0, rtol=0, atol=1e-14)   # probabilities sum to 1
    v = rng.standard_normal((2, 2, 1, 4))
    got = A.gated_attention(q[:, :, :1], k[:, :, :1], v, 0.7)
    assert np.allclose(got, np.transpose(v, (0, 2, 1, 3)).reshape(2, 1, 8), rtol=0, atol=1e-15)


def test_narrow_v_is_the_wide_result_restricted():
    """The output is linear in v column by column: v narrower than q gives exactly the first columns
    of the output for a wider v that starts with the same columns (a dropped or shifted v column, or
    a dqk/dv mix-up in the head stride, fails this)."""
    rng = np.random.default_rng(2)
    S, H, n, dqk = 2, 3, 9, 8
    q, k = rng.standard_normal((S, H, n, dqk)), rng.standard_normal((S, H, n, dqk))
    vw = rng.standard_normal((S, H, n, dqk))
    wide = A.gated_attention(q, k, vw, 0.3).reshape(S, n, H, dqk)
    narrow = A.gated_attention(q, k, vw[..., :3], 0.3).reshape(S, n, H, 3)
    assert np.allclose(narrow, wide[..., :3], rtol=0, atol=1e-14)


def test_zero_queries_average_the_values():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((1, 2, 6, 3))
    got = A.gated_attention(np.zeros((1, 2, 6, 8)), rng.standard_normal((1, 2, 6, 8)), v, 1.0)
    want = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    assert np.allclose(got, np.transpose(want, (0, 2, 1, 3)).reshape(1, 6, 6), rtol=0, atol=1e-14)
