"""A second, independent statement of the core in scalar Python loops (test infrastructure).

It exists to pin ``oracle.model``: the two share no helper (no numpy algebra here, no
table builder), so a dropped term, a transposed operand or a wrong index in either
shows up as a disagreement on tiny shapes.  Every step follows the same passages
``oracle.model`` cites; membership in a band is taken from the closed form of the
triangle (weight > 0 exactly when the bin frequency lies strictly between the
band's outer mel points) instead of evaluating and thresholding weights.

Only meant for tiny configurations (a few hundred tokens of width 8).
"""
from __future__ import annotations

import math
from typing import Dict, List


def _hz_to_mel(f: float) -> float:
    # Slaney: 3 mels per 200 Hz up to 1 kHz (= 15 mels), then 27 mels per factor 6.4
    if f < 1000.0:
        return 3.0 * f / 200.0
    return 15.0 + 27.0 * math.log(f / 1000.0) / math.log(6.4)


def _mel_to_hz(m: float) -> float:
    if m < 15.0:
        return 200.0 * m / 3.0
    return 1000.0 * math.exp((m - 15.0) * math.log(6.4) / 27.0)


def bands(sample_rate: int, n_fft: int, n_bands: int) -> List[List[int]]:
    """Ascending bins of each band: strictly inside the band's outer mel points, plus
    DC forced into the first band and Nyquist into the last."""
    n_freqs = n_fft // 2 + 1
    top = _hz_to_mel(sample_rate / 2.0)
    pts = [_mel_to_hz(top * j / (n_bands + 1)) for j in range(n_bands + 2)]
    out = []
    for i in range(n_bands):
        lo, hi = pts[i], pts[i + 2]
        members = [k for k in range(n_freqs) if lo < k * sample_rate / n_fft < hi]
        if i == 0 and 0 not in members:
            members = [0] + members
        if i == n_bands - 1 and (n_freqs - 1) not in members:
            members = members + [n_freqs - 1]
        out.append(members)
    return out


def _norm(v: List[float], gamma: List[float]) -> List[float]:
    s = math.sqrt(sum(a * a for a in v))
    den = max(s, 1e-12)
    r = math.sqrt(len(v))
    return [v[e] / den * r * gamma[e] for e in range(len(v))]


def _linear(v: List[float], W, bias=None) -> List[float]:
    """W is [out][in] (array-like indexed elementwise)."""
    out = []
    for o in range(len(W)):
        acc = 0.0 if bias is None else float(bias[o])
        for e in range(len(v)):
            acc += v[e] * float(W[o][e])
        out.append(acc)
    return out


def _gelu(a: float) -> float:
    return 0.5 * a * (1.0 + math.erf(a / math.sqrt(2.0)))


def _sig(a: float) -> float:
    return 1.0 / (1.0 + math.exp(-a))


def _transformer(seq: List[List[float]], w: Dict, p: str, heads: int, dh: int) -> List[List[float]]:
    n = len(seq)
    I = heads * dh
    xn = [_norm(v, w[p + "attn.norm.gamma"]) for v in seq]
    qkv = [_linear(v, w[p + "attn.to_qkv.weight"]) for v in xn]
    q = [[[qkv[t][h * dh + d] for d in range(dh)] for t in range(n)] for h in range(heads)]
    k = [[[qkv[t][I + h * dh + d] for d in range(dh)] for t in range(n)] for h in range(heads)]
    v = [[[qkv[t][2 * I + h * dh + d] for d in range(dh)] for t in range(n)] for h in range(heads)]
    for h in range(heads):
        for t in range(n):
            for j in range(dh // 2):
                ang = t * math.pow(10000.0, -2.0 * j / dh)
                c, s = math.cos(ang), math.sin(ang)
                for vec in (q[h][t], k[h][t]):
                    a, b = vec[2 * j], vec[2 * j + 1]
                    vec[2 * j], vec[2 * j + 1] = a * c - b * s, a * s + b * c
    gate = [[_sig(g) for g in _linear(xn[t], w[p + "attn.to_gates.weight"], w[p + "attn.to_gates.bias"])]
            for t in range(n)]
    cat = [[0.0] * I for _ in range(n)]
    for h in range(heads):
        for i in range(n):
            sc = [sum(q[h][i][d] * k[h][j][d] for d in range(dh)) / math.sqrt(dh) for j in range(n)]
            m = max(sc)
            e = [math.exp(x - m) for x in sc]
            z = sum(e)
            for d in range(dh):
                cat[i][h * dh + d] = sum(e[j] / z * v[h][j][d] for j in range(n)) * gate[i][h]
    x1 = []
    for t in range(n):
        upd = _linear(cat[t], w[p + "attn.to_out.weight"])
        x1.append([seq[t][d] + upd[d] for d in range(len(upd))])
    x2 = []
    for t in range(n):
        hid = [_gelu(a) for a in _linear(_norm(x1[t], w[p + "ff.norm.gamma"]), w[p + "ff.fc1.weight"], w[p + "ff.fc1.bias"])]
        out = _linear(hid, w[p + "ff.fc2.weight"], w[p + "ff.fc2.bias"])
        x2.append([x1[t][d] + out[d] for d in range(len(out))])
    return [_norm(vv, w[p + "norm.gamma"]) for vv in x2]


def forward(spec, sample_rate: int, n_fft: int, channels: int, n_bands: int, dim: int, depth: int,
            heads: int, dh: int, mask_depth: int, w: Dict, stem: int = 0):
    """spec [B, F*S, T, 2] (array-like) -> masks as nested lists [B][F*S][T][2]."""
    B, T = len(spec), len(spec[0][0])
    S = channels
    n_freqs = n_fft // 2 + 1
    bl = bands(sample_rate, n_fft, n_bands)
    # band embedding
    x = [[[None] * n_bands for _ in range(T)] for _ in range(B)]
    for b in range(B):
        for t in range(T):
            for i in range(n_bands):
                feats = [float(spec[b][k * S + s][t][c]) for k in bl[i] for s in range(S) for c in range(2)]
                u = _norm(feats, w[f"band{i}.norm.gamma"])
                x[b][t][i] = _linear(u, w[f"band{i}.proj.weight"], w[f"band{i}.proj.bias"])
    for l in range(depth):
        for b in range(B):
            for i in range(n_bands):
                out = _transformer([x[b][t][i] for t in range(T)], w, f"layer{l}.time.", heads, dh)
                for t in range(T):
                    x[b][t][i] = out[t]
        for b in range(B):
            for t in range(T):
                x[b][t] = _transformer(x[b][t], w, f"layer{l}.band.", heads, dh)
    # mask head and average
    acc = [[[[0.0, 0.0] for _ in range(T)] for _ in range(n_freqs * S)] for _ in range(B)]
    cnt = [sum(1 for i in range(n_bands) if k in bl[i]) for k in range(n_freqs)]
    for i in range(n_bands):
        W = 2 * S * len(bl[i])
        for b in range(B):
            for t in range(T):
                h = x[b][t][i]
                for j in range(mask_depth + 1):
                    pre = f"stem{stem}.band{i}.mlp{j}."
                    h = _linear(h, w[pre + "weight"], w[pre + "bias"])
                    if j < mask_depth:
                        h = [math.tanh(a) for a in h]
                m = [h[e] * _sig(h[W + e]) for e in range(W)]
                for r, k in enumerate(bl[i]):
                    for s in range(S):
                        for c in range(2):
                            acc[b][k * S + s][t][c] += m[(r * S + s) * 2 + c]
    for b in range(B):
        for k in range(n_freqs):
            for s in range(S):
                for t in range(T):
                    for c in range(2):
                        acc[b][k * S + s][t][c] /= cnt[k]
    return acc
