"""Gated scaled dot-product attention with queries and keys wider than the values (oracle, fp64,
test infrastructure only).

[P2] "Evaluation record", section "BS PolarFormer: the same quality for a quarter of the
arithmetic", part "Ported, and what it actually bought": the polar positional scheme doubles the
depth of q and k while v keeps its width, so a fused attention has to accept v narrower than q.
The positional transform itself is not on the pages; here q and k arrive already transformed (an
identity positional map), and the attention is the plain definition:

    o[s, h, t, :] = gate[s, t, h] * sum_j softmax_j(scale * q[s, h, t, :] . k[s, h, j, :]) v[s, h, j, :]

with q, k of width dqk and v of width dv (any dv), the softmax over all n keys with no mask
([P1] "Per Attention layer": per head, times that head's gate).
"""
from __future__ import annotations

import numpy as np


def gated_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    gates: np.ndarray | None = None) -> np.ndarray:
    """q, k [S, H, n, dqk], v [S, H, n, dv], gates [S, n, H] or None -> o [S, n, H * dv].
    The softmax subtracts each row's max before the exponential (exact in real arithmetic)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    S, H, n, _ = q.shape
    dv = v.shape[-1]
    o = np.empty((S, H, n, dv))
    for s in range(S):                                    # bounds the [H, n, n] scores
        sc = (q[s] @ np.swapaxes(k[s], -1, -2)) * scale
        sc = sc - sc.max(axis=-1, keepdims=True)
        p = np.exp(sc)
        p = p / p.sum(axis=-1, keepdims=True)
        o[s] = p @ v[s]
    if gates is not None:
        o = o * np.transpose(np.asarray(gates, np.float64), (0, 2, 1))[..., None]
    return np.transpose(o, (0, 2, 1, 3)).reshape(S, n, H * dv)
