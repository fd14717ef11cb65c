"""The Mel-Band RoFormer core in fp64 numpy (oracle, test infrastructure only).

What is computed, step by step, and where each step is stated:

 1. Band tables: ``oracle.mel`` ([P1] "The mel-band split, exactly").
 2. Band embedding: the gathered complex stereo values of a band, re/im folded into
    features as (pair rank, re/im), RMSNorm over the band's features, then the band's
    own Linear(W_i, D) with bias ([P1] "The forward chain" and the BandSplit paragraph;
    [P5] export-roformer.py, Core.build, band split tables and ``forward``).
 3. For each of ``depth`` axial blocks: a Transformer along time (one sequence per
    (batch, band), positions = frames), then a Transformer along the bands (one
    sequence per (batch, frame), positions = band index) ([P1] "The two transformers
    are not the same shape"; [P5] ``forward``: time then frequency per depth).
    Each Transformer: x += Attn(x); x += FF(x); x = RMSNorm_out(x)
    ([P5] export-roformer.py, class Block).
      Attn ([P1] "Per Attention layer"; [P5] class Attn): x^ = RMSNorm(x);
      q, k, v = x^ W_qkv^T split head-major; rotary on q and k; per head
      softmax(q k^T / sqrt(dh)) v; times sigmoid(x^ W_g^T + b_g) per head; W_out.
      FF ([P5] class FF): W_2 GELU(RMSNorm(x) W_1^T + b_1) + b_2, exact-erf GELU.
 4. Mask head per stem and band ([P1] "Parameter accounting": Linear(D, MH), Tanh,
    Linear(MH, MH), Tanh, Linear(MH, 2 W_i), GLU); GLU keeps the first half times
    the sigmoid of the second ([P5] ``forward``: value half first).
 5. Average: each band's mask features are scattered back to their (pair, re/im)
    and divided by the number of bands covering the bin ([P1] "The forward chain":
    scatter_add_ then divide by num_bands_per_freq).

RMSNorm everywhere: x / max(||x||_2, 1e-12) * sqrt(d) * gamma ([P1] the RMSNorm
paragraph under BandSplit: F.normalize times sqrt(dim) times gamma).

Readings where the pages are silent (parity unpinned against the real model):
rotary base 10000 with inverse frequencies base^(-2j/dh) over interleaved pairs
(2j, 2j+1), positions 0..n-1 per call; attention scale dh^-1/2.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, List, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf

from . import mel

KIND_MATRIX, KIND_BIAS, KIND_GAMMA = 0, 1, 2
NORM_EPS = 1e-12
ROPE_BASE = 10000.0
_WORKERS = max(1, min(16, os.cpu_count() or 1))


@dataclass(frozen=True)
class CoreConfig:
    sample_rate: int
    n_fft: int
    audio_channels: int
    num_bands: int
    dim: int
    depth: int
    heads: int
    dim_head: int
    ff_mult: int = 4
    mask_hidden_mult: int = 4
    mask_depth: int = 2
    num_stems: int = 1
    zero_dc: bool = False                 # the DC bin's masks set to zero ([P5] export-roformer.py option)
    band_bins: Tuple[int, ...] | None = None   # explicit non-overlapping band table (None: mel)

    @property
    def inner(self) -> int:
        return self.heads * self.dim_head

    @property
    def ff(self) -> int:
        return self.ff_mult * self.dim

    @property
    def mask_hidden(self) -> int:
        return self.mask_hidden_mult * self.dim

    def tables(self) -> mel.BandTables:
        if self.band_bins is not None:
            if len(self.band_bins) != self.num_bands:
                raise ValueError("band_bins needs one count per band")
            return mel.explicit_band_tables(self.n_fft, self.band_bins, self.audio_channels)
        return mel.band_tables(self.sample_rate, self.n_fft, self.num_bands, self.audio_channels)


# ----------------------------------------------------------------------------- inventory

def inventory(cfg: CoreConfig) -> List[Tuple[str, Tuple[int, ...], int]]:
    """Every parameter of the core in canonical order: (name, shape, kind).

    Shapes follow the module tree the pages describe ([P1] "Parameter accounting":
    to_qkv Linear(dim, 3*heads*dim_head, no bias), to_gates Linear(dim, heads) with
    bias, to_out Linear(heads*dim_head, dim, no bias); BandSplit RMSNorm(W_i) +
    Linear(W_i, dim); FeedForward RMSNorm + Linear(dim, ff) + Linear(ff, dim), both
    with bias; one output RMSNorm per Transformer; mask MLP per band and stem).
    Linear weights are [out, in].
    """
    t = cfg.tables()
    D, I, H, FF, MH = cfg.dim, cfg.inner, cfg.heads, cfg.ff, cfg.mask_hidden
    inv: List[Tuple[str, Tuple[int, ...], int]] = []
    for i, W in enumerate(t.widths.tolist()):
        inv += [(f"band{i}.norm.gamma", (W,), KIND_GAMMA),
                (f"band{i}.proj.weight", (D, W), KIND_MATRIX),
                (f"band{i}.proj.bias", (D,), KIND_BIAS)]
    for l in range(cfg.depth):
        for axis in ("time", "band"):
            p = f"layer{l}.{axis}."
            inv += [(p + "attn.norm.gamma", (D,), KIND_GAMMA),
                    (p + "attn.to_qkv.weight", (3 * I, D), KIND_MATRIX),
                    (p + "attn.to_gates.weight", (H, D), KIND_MATRIX),
                    (p + "attn.to_gates.bias", (H,), KIND_BIAS),
                    (p + "attn.to_out.weight", (D, I), KIND_MATRIX),
                    (p + "ff.norm.gamma", (D,), KIND_GAMMA),
                    (p + "ff.fc1.weight", (FF, D), KIND_MATRIX),
                    (p + "ff.fc1.bias", (FF,), KIND_BIAS),
                    (p + "ff.fc2.weight", (D, FF), KIND_MATRIX),
                    (p + "ff.fc2.bias", (D,), KIND_BIAS),
                    (p + "norm.gamma", (D,), KIND_GAMMA)]
    for s in range(cfg.num_stems):
        for i, W in enumerate(t.widths.tolist()):
            dims = [D] + [MH] * cfg.mask_depth + [2 * W]
            for j in range(len(dims) - 1):
                p = f"stem{s}.band{i}.mlp{j}."
                inv += [(p + "weight", (dims[j + 1], dims[j]), KIND_MATRIX),
                        (p + "bias", (dims[j + 1],), KIND_BIAS)]
    return inv


def param_count(cfg: CoreConfig) -> int:
    return int(sum(np.prod(s) for _, s, _ in inventory(cfg)))


def named(cfg: CoreConfig, weights: Sequence[np.ndarray]) -> Dict[str, np.ndarray]:
    inv = inventory(cfg)
    if len(weights) != len(inv):
        raise ValueError(f"expected {len(inv)} tensors, got {len(weights)}")
    out = {}
    for (name, shape, _), w in zip(inv, weights):
        w = np.asarray(w, dtype=np.float64)
        if tuple(w.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {w.shape}, expected {shape}")
        out[name] = w
    return out


# ----------------------------------------------------------------------------- layouts

def read_input(x: np.ndarray, channels: int, layout: int) -> np.ndarray:
    """Either boundary layout to [B, F*S, T, 2] fp64.

    layout 0: [B, F*S, T, 2], pair = f*S + s, last axis (re, im) ([P3] signature table).
    layout 1: [B, S*2, F, T], planes (L re, L im, R re, R im) ([P4] "Graph").
    """
    x = np.asarray(x, dtype=np.float64)
    if layout == 0:
        return x
    B, SC, F, T = x.shape
    S = channels
    y = x.reshape(B, S, 2, F, T)                       # [b, s, c, f, t]
    y = np.transpose(y, (0, 3, 1, 4, 2))               # [b, f, s, t, c]
    return y.reshape(B, F * S, T, 2)


def write_output(m: np.ndarray, channels: int, layout: int) -> np.ndarray:
    """[B, F*S, T, 2] masks to the boundary layout (the inverse of ``read_input``)."""
    if layout == 0:
        return m
    B, FS, T, _ = m.shape
    S = channels
    F = FS // S
    y = m.reshape(B, F, S, T, 2)
    y = np.transpose(y, (0, 2, 4, 1, 3))               # [b, s, c, f, t]
    return y.reshape(B, S * 2, F, T)


# ----------------------------------------------------------------------------- steps

def rmsnorm(x: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    """x / max(||x||, 1e-12) * sqrt(d) * gamma over the last axis ([P1] RMSNorm paragraph)."""
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, NORM_EPS) * math.sqrt(x.shape[-1]) * gamma


def _gelu_block(x: np.ndarray) -> np.ndarray:
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU, x * Phi(x) with the error function ([P5] class FF uses F.gelu).
    The error function is scipy's (a library primitive; pinned against math.erf).  Large arrays
    are evaluated in row blocks on a thread pool; every element is computed the same way."""
    if x.size < (1 << 20):
        return _gelu_block(x)
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty_like(flat)
    step = max(1, flat.shape[0] // (4 * _WORKERS))

    def run(a):
        out[a:a + step] = _gelu_block(flat[a:a + step])

    with ThreadPoolExecutor(_WORKERS) as ex:
        list(ex.map(run, range(0, flat.shape[0], step)))
    return out.reshape(x.shape)


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def gather_band_inputs(spec: np.ndarray, tables: mel.BandTables) -> List[np.ndarray]:
    """Per band: [B, T, W_i] with feature = (rank of the pair within the band)*2 + (re, im)
    ([P1] "The forward chain": gather by mel band, fold the complex axis into channels)."""
    B, _, T, _ = spec.shape
    out = []
    for pairs in tables.pairs:
        v = spec[:, pairs, :, :]                       # [B, P_i, T, 2]
        out.append(np.transpose(v, (0, 2, 1, 3)).reshape(B, T, 2 * len(pairs)))
    return out


def band_embed(spec: np.ndarray, cfg: CoreConfig, w: Dict[str, np.ndarray], tables: mel.BandTables) -> np.ndarray:
    """[B, F*S, T, 2] -> x [B, T, NB, D]: per band RMSNorm(W_i) then Linear(W_i, D) with bias."""
    xs = []
    for i, v in enumerate(gather_band_inputs(spec, tables)):
        u = rmsnorm(v, w[f"band{i}.norm.gamma"])
        xs.append(u @ w[f"band{i}.proj.weight"].T + w[f"band{i}.proj.bias"])
    return np.stack(xs, axis=2)


def rope_angles(n: int, dh: int) -> np.ndarray:
    """[n, dh/2] angles pos * base^(-2j/dh), positions 0..n-1 (rotary embedding of dim dh)."""
    j = np.arange(dh // 2, dtype=np.float64)
    inv_freq = ROPE_BASE ** (-2.0 * j / dh)
    return np.arange(n, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs (x[2j], x[2j+1]) of the last axis by angles[pos, j];
    x is [..., n, dh]."""
    c, s = np.cos(angles), np.sin(angles)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def softmax(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention(xs: np.ndarray, cfg: CoreConfig, w: Dict[str, np.ndarray], p: str, chunk: int = 0) -> np.ndarray:
    """Gated multi-head attention over sequences xs [S, n, D] -> [S, n, D] (the update,
    before the residual add) ([P1] "Per Attention layer"; [P5] class Attn)."""
    S, n, D = xs.shape
    H, dh, I = cfg.heads, cfg.dim_head, cfg.inner
    xn = rmsnorm(xs, w[p + "attn.norm.gamma"])
    qkv = xn @ w[p + "attn.to_qkv.weight"].T                      # [S, n, 3I]
    q = qkv[..., 0 * I:1 * I].reshape(S, n, H, dh).transpose(0, 2, 1, 3)
    k = qkv[..., 1 * I:2 * I].reshape(S, n, H, dh).transpose(0, 2, 1, 3)
    v = qkv[..., 2 * I:3 * I].reshape(S, n, H, dh).transpose(0, 2, 1, 3)
    ang = rope_angles(n, dh)
    q, k = rope(q, ang), rope(k, ang)
    scale = dh ** -0.5
    o = np.empty_like(q)                                          # [S, H, n, dh]
    step = chunk if chunk > 0 else S
    for a in range(0, S, step):                                   # bounds the [step, H, n, n] scores
        sc = (q[a:a + step] @ np.swapaxes(k[a:a + step], -1, -2)) * scale
        o[a:a + step] = softmax(sc) @ v[a:a + step]
    g = sigmoid(xn @ w[p + "attn.to_gates.weight"].T + w[p + "attn.to_gates.bias"])   # [S, n, H]
    o = o * g.transpose(0, 2, 1)[..., None]
    o = o.transpose(0, 2, 1, 3).reshape(S, n, I)
    return o @ w[p + "attn.to_out.weight"].T


def feed_forward(xs: np.ndarray, w: Dict[str, np.ndarray], p: str) -> np.ndarray:
    h = rmsnorm(xs, w[p + "ff.norm.gamma"]) @ w[p + "ff.fc1.weight"].T + w[p + "ff.fc1.bias"]
    return gelu(h) @ w[p + "ff.fc2.weight"].T + w[p + "ff.fc2.bias"]


def transformer(xs: np.ndarray, cfg: CoreConfig, w: Dict[str, np.ndarray], p: str, chunk: int = 0) -> np.ndarray:
    """One Transformer over [S, n, D]: attention, feed-forward, output RMSNorm ([P5] class Block)."""
    xs = xs + attention(xs, cfg, w, p, chunk)
    xs = xs + feed_forward(xs, w, p)
    return rmsnorm(xs, w[p + "norm.gamma"])


def time_transformer(x: np.ndarray, cfg, w, p, chunk=0) -> np.ndarray:
    """x [B, T, NB, D]: sequences (b, band) along frames."""
    B, T, NB, D = x.shape
    xs = x.transpose(0, 2, 1, 3).reshape(B * NB, T, D)
    xs = transformer(xs, cfg, w, p, chunk)
    return xs.reshape(B, NB, T, D).transpose(0, 2, 1, 3)


def band_transformer(x: np.ndarray, cfg, w, p, chunk=0) -> np.ndarray:
    """x [B, T, NB, D]: sequences (b, frame) along bands."""
    B, T, NB, D = x.shape
    xs = transformer(x.reshape(B * T, NB, D), cfg, w, p, chunk)
    return xs.reshape(B, T, NB, D)


def mask_head(x: np.ndarray, cfg: CoreConfig, w: Dict[str, np.ndarray], tables: mel.BandTables, stem: int) -> List[np.ndarray]:
    """Per band: m_i [B, T, W_i] = GLU(MLP_i(x[:, :, i])) ([P1] "Parameter accounting")."""
    out = []
    for i, W in enumerate(tables.widths.tolist()):
        h = x[:, :, i, :]
        nl = cfg.mask_depth + 1
        for j in range(nl):
            p = f"stem{stem}.band{i}.mlp{j}."
            h = h @ w[p + "weight"].T + w[p + "bias"]
            if j < nl - 1:
                h = np.tanh(h)
        out.append(h[..., :W] * sigmoid(h[..., W:]))
    return out


def average(masks: List[np.ndarray], tables: mel.BandTables, zero_dc: bool = False) -> np.ndarray:
    """Scatter-add each band's features back to (pair, re/im), divide by the bin's band count;
    with zero_dc the DC bin's masks are zero.  Returns [B, F*S, T, 2]."""
    B, T, _ = masks[0].shape
    S = tables.channels
    out = np.zeros((B, tables.n_freqs * S, T, 2))
    for m, pairs in zip(masks, tables.pairs):
        out[:, pairs, :, :] += np.transpose(m.reshape(B, T, len(pairs), 2), (0, 2, 1, 3))
    per_pair = np.repeat(tables.counts, S).astype(np.float64)
    out = out / per_pair[None, :, None, None]
    if zero_dc:
        out[:, :S] = 0.0
    return out


@dataclass
class Taps:
    embed: np.ndarray = None
    after: List[np.ndarray] = None       # x after each Transformer, [B, T, NB, D]
    glu: List[np.ndarray] = None         # per band m_i of stem 0


def forward(spec_in: np.ndarray, cfg: CoreConfig, weights: Sequence[np.ndarray], layout: int = 0,
            taps: Taps | None = None, chunk: int = 64) -> np.ndarray:
    """The whole core: stft_repr -> masks, in the boundary layout.

    Returns [B, F*S, T, 2] (layout 0) or [B, S*2, F, T] (layout 1) for one stem, and a
    leading stem axis after B when num_stems > 1.
    """
    tables = cfg.tables()
    w = named(cfg, weights)
    spec = read_input(spec_in, cfg.audio_channels, layout)
    x = band_embed(spec, cfg, w, tables)
    if taps is not None:
        taps.embed = x.copy()
        taps.after = []
    for l in range(cfg.depth):
        x = time_transformer(x, cfg, w, f"layer{l}.time.", chunk=1)
        if taps is not None:
            taps.after.append(x.copy())
        x = band_transformer(x, cfg, w, f"layer{l}.band.", chunk=chunk)
        if taps is not None:
            taps.after.append(x.copy())
    outs = []
    for s in range(cfg.num_stems):
        m = mask_head(x, cfg, w, tables, s)
        if taps is not None and s == 0:
            taps.glu = m
        outs.append(write_output(average(m, tables, cfg.zero_dc), cfg.audio_channels, layout))
    return outs[0] if cfg.num_stems == 1 else np.stack(outs, axis=1)
