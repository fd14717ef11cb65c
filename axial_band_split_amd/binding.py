"""Thin ctypes binding of libmbr_core.so: the C entry points under the same names, plus argument
marshalling helpers.  Every step of the forward runs in the library's HIP kernels; torch is used
only to hold device memory and to name streams.  There is no fallback: if the library is missing
or does not load, ``lib()`` raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Sequence, Tuple

import numpy as np

from . import synth

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmbr_core.so")

MBR_OK, MBR_E_ARG, MBR_E_CONFIG, MBR_E_DEVICE, MBR_E_HIP, MBR_E_NOMEM = 0, -1, -2, -3, -4, -5
MBR_ISTFT_NOALLOC_MAX_BYTES = 64 << 20       # the static frame buffer of mbr_istft_masked_noalloc

# Every symbol include/mbr_core.h declares, with (restype, argtypes).
_SIGS = {
    "mbr_last_error": (C.c_char_p, []),
    "mbr_core_weight_count": (C.c_int, [C.c_void_p]),
    "mbr_core_weight_info": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_int), C.POINTER(C.c_int64), C.POINTER(C.c_int)]),
    "mbr_core_table_sizes": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "mbr_core_tables": (C.c_int, [C.c_void_p] + [C.c_void_p] * 6),
    "mbr_core_create": (C.c_int, [C.c_void_p, C.POINTER(C.c_void_p), C.c_int, C.POINTER(C.c_void_p)]),
    "mbr_core_forward": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_void_p]),
    "mbr_core_destroy": (None, [C.c_void_p]),
    "mbr_core_debug_size": (C.c_int64, [C.c_void_p, C.c_int, C.c_int]),
    "mbr_core_forward_debug": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p]),
    "mbr_core_forward_profiled": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_void_p,
                                            C.POINTER(C.c_double), C.POINTER(C.c_int32)]),
    "mbr_core_device_bytes": (C.c_int64, [C.c_void_p]),
    "mbr_k_gemm": (C.c_int, [C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                             C.c_int, C.c_int, C.c_void_p]),
    "mbr_k_gemm_variants": (C.c_int, []),
    "mbr_k_gelu": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_void_p]),
    "mbr_attention": (C.c_int, [C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                                C.c_int, C.c_int, C.c_int, C.c_int, C.c_float, C.c_void_p]),
    "mbr_stft": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_int, C.c_int, C.c_void_p, C.c_void_p]),
    "mbr_istft_workspace_size": (C.c_int64, [C.c_int, C.c_int, C.c_int, C.c_int]),
    "mbr_istft_masked": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int64, C.c_int, C.c_int, C.c_void_p,
                                   C.c_void_p, C.c_void_p]),
    "mbr_istft_masked_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int64, C.c_int, C.c_int,
                                           C.c_void_p, C.c_void_p]),
    "mbr_separate_workspace_size": (C.c_int64, [C.c_void_p, C.c_int64, C.c_int]),
    "mbr_separate": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]),
    "mbr_separate_workspace_size_strided": (C.c_int64, [C.c_void_p, C.c_int64, C.c_int, C.c_int64]),
    "mbr_separate_strided": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int, C.c_int64, C.c_void_p, C.c_void_p,
                                       C.c_void_p]),
}
KERNEL_KINDS = ("gather", "embed", "norm", "qkv", "attn_time", "attn_band", "out_proj", "ffn1", "ffn2",
                "mask_hidden", "mask_glu", "average", "block", "band_attn")
SYMBOLS = tuple(_SIGS)


class MbrConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "sample_rate", "n_fft", "audio_channels", "num_bands", "dim", "depth", "heads", "dim_head", "ff_mult",
        "mask_hidden_mult", "mask_depth", "num_stems", "max_batch", "frames", "dtype", "io_layout", "zero_dc")] + [
        ("band_bins", C.POINTER(C.c_int32))]


class MbrError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mbr error {code}: {msg}")
        self.code = code


_LIB = None


def lib() -> C.CDLL:
    """Load libmbr_core.so (built in-tree by axial_band_split_amd.build); raise if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(f"{LIB_PATH} is missing: build it with python -m axial_band_split_amd.build")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _LIB = h
    return _LIB


def _check(rc: int) -> int:
    if rc < 0:
        raise MbrError(rc, mbr_last_error())
    return rc


def config(w: synth.Workload, max_batch: int | None = None, **override) -> MbrConfig:
    vals = dict(sample_rate=w.sample_rate, n_fft=w.n_fft, audio_channels=w.audio_channels, num_bands=w.num_bands,
                dim=w.dim, depth=w.depth, heads=w.heads, dim_head=w.dim_head, ff_mult=w.ff_mult,
                mask_hidden_mult=w.mask_hidden_mult, mask_depth=w.mask_depth, num_stems=w.num_stems,
                max_batch=w.batch if max_batch is None else max_batch, frames=w.frames, dtype=w.dtype,
                io_layout=w.io_layout, zero_dc=w.zero_dc, band_bins=w.band_bins)
    vals.update(override)
    bins = vals.pop("band_bins")
    cfg = MbrConfig(**vals)
    if bins is not None:
        arr = (C.c_int32 * len(bins))(*bins)
        cfg._bins = arr                      # kept alive with the structure
        cfg.band_bins = C.cast(arr, C.POINTER(C.c_int32))
    return cfg


# ----------------------------------------------------------------------------- C entry points

def mbr_last_error() -> str:
    return lib().mbr_last_error().decode()


def mbr_core_weight_count(cfg: MbrConfig) -> int:
    return _check(lib().mbr_core_weight_count(C.byref(cfg)))


def mbr_core_weight_info(cfg: MbrConfig, index: int) -> Tuple[Tuple[int, ...], int]:
    nd, kind = C.c_int(), C.c_int()
    dims = (C.c_int64 * 2)()
    _check(lib().mbr_core_weight_info(C.byref(cfg), index, C.byref(nd), dims, C.byref(kind)))
    shape = (dims[0],) if nd.value == 1 else (dims[0], dims[1])
    return shape, kind.value


def mbr_core_table_sizes(cfg: MbrConfig) -> Tuple[int, int, int]:
    nb, tw, nf = C.c_int32(), C.c_int32(), C.c_int32()
    _check(lib().mbr_core_table_sizes(C.byref(cfg), C.byref(nb), C.byref(tw), C.byref(nf)))
    return nb.value, tw.value, nf.value


def mbr_core_tables(cfg: MbrConfig) -> dict:
    nb, tw, nf = mbr_core_table_sizes(cfg)
    S = cfg.audio_channels
    out = dict(band_bins=np.zeros(nb, np.int32), band_offset=np.zeros(nb + 1, np.int32),
               gather_pair=np.zeros(tw // 2, np.int32), inv_slot=np.zeros(nf * S * 2, np.int32),
               inv_weight=np.zeros(nf * S, np.float32), bin_count=np.zeros(nf, np.int32))
    ptrs = [a.ctypes.data_as(C.c_void_p) for a in out.values()]
    _check(lib().mbr_core_tables(C.byref(cfg), *ptrs))
    return out


def mbr_core_create(cfg: MbrConfig, weight_ptrs: Sequence[int]) -> C.c_void_p:
    arr = (C.c_void_p * len(weight_ptrs))(*[C.c_void_p(p) for p in weight_ptrs])
    h = C.c_void_p()
    _check(lib().mbr_core_create(C.byref(cfg), arr, len(weight_ptrs), C.byref(h)))
    return h


def mbr_core_forward(h, stft_repr_ptr: int, masks_ptr: int, batch: int, stream_ptr: int = 0) -> None:
    _check(lib().mbr_core_forward(h, C.c_void_p(stft_repr_ptr), C.c_void_p(masks_ptr), batch, C.c_void_p(stream_ptr)))


def mbr_core_destroy(h) -> None:
    lib().mbr_core_destroy(h)


def mbr_core_debug_size(h, batch: int, stage: int) -> int:
    return _check(lib().mbr_core_debug_size(h, batch, stage))


def mbr_core_forward_debug(h, stft_repr_ptr: int, batch: int, stage: int, out_ptr: int, stream_ptr: int = 0) -> None:
    _check(lib().mbr_core_forward_debug(h, C.c_void_p(stft_repr_ptr), batch, stage, C.c_void_p(out_ptr),
                                        C.c_void_p(stream_ptr)))


def mbr_core_forward_profiled(h, stft_repr_ptr: int, masks_ptr: int, batch: int, stream_ptr: int = 0):
    """Returns {kind: (milliseconds summed over launches, launches)} for one forward."""
    ms = (C.c_double * len(KERNEL_KINDS))()
    n = (C.c_int32 * len(KERNEL_KINDS))()
    _check(lib().mbr_core_forward_profiled(h, C.c_void_p(stft_repr_ptr), C.c_void_p(masks_ptr), batch,
                                           C.c_void_p(stream_ptr), ms, n))
    return {k: (ms[i], n[i]) for i, k in enumerate(KERNEL_KINDS)}


def mbr_core_device_bytes(h) -> int:
    return lib().mbr_core_device_bytes(h)


def mbr_k_gemm(dtype: int, a_ptr: int, b_ptr: int, bias_ptr: int, c_ptr: int, M: int, N: int, K: int, variant: int = 0,
               out16: bool = False, stream_ptr: int = 0) -> None:
    _check(lib().mbr_k_gemm(dtype, C.c_void_p(a_ptr), C.c_void_p(b_ptr), C.c_void_p(bias_ptr or None),
                            C.c_void_p(c_ptr), M, N, K, variant, int(out16), C.c_void_p(stream_ptr)))


def mbr_k_gelu(x_ptr: int, y_ptr: int, n: int, stream_ptr: int = 0) -> None:
    _check(lib().mbr_k_gelu(C.c_void_p(x_ptr), C.c_void_p(y_ptr), n, C.c_void_p(stream_ptr)))


def mbr_attention(dtype: int, q_ptr: int, k_ptr: int, vt_ptr: int, gates_ptr: int, o_ptr: int, seqs: int, heads: int,
                  n: int, npad: int, dqk: int, dv: int, scale: float, stream_ptr: int = 0) -> None:
    _check(lib().mbr_attention(dtype, C.c_void_p(q_ptr), C.c_void_p(k_ptr), C.c_void_p(vt_ptr),
                               C.c_void_p(gates_ptr or None), C.c_void_p(o_ptr), seqs, heads, n, npad, dqk, dv,
                               scale, C.c_void_p(stream_ptr)))


def mbr_stft(wave_ptr: int, channels: int, length: int, n_fft: int, hop: int, spec_ptr: int, stream_ptr: int = 0) -> None:
    _check(lib().mbr_stft(C.c_void_p(wave_ptr), channels, length, n_fft, hop, C.c_void_p(spec_ptr), C.c_void_p(stream_ptr)))


def mbr_istft_workspace_size(channels: int, n_fft: int, frames: int, stems: int) -> int:
    return _check(lib().mbr_istft_workspace_size(channels, n_fft, frames, stems))


def mbr_istft_masked(spec_ptr: int, masks_ptr: int, stems: int, channels: int, length: int, n_fft: int, hop: int,
                     ws_ptr: int, out_ptr: int, stream_ptr: int = 0) -> None:
    _check(lib().mbr_istft_masked(C.c_void_p(spec_ptr), C.c_void_p(masks_ptr), stems, channels, length, n_fft, hop,
                                  C.c_void_p(ws_ptr), C.c_void_p(out_ptr), C.c_void_p(stream_ptr)))


def mbr_istft_masked_noalloc(spec_ptr: int, masks_ptr: int, stems: int, channels: int, length: int, n_fft: int,
                             hop: int, out_ptr: int, stream_ptr: int = 0) -> None:
    _check(lib().mbr_istft_masked_noalloc(C.c_void_p(spec_ptr), C.c_void_p(masks_ptr), stems, channels, length, n_fft,
                                          hop, C.c_void_p(out_ptr), C.c_void_p(stream_ptr)))


def mbr_separate_workspace_size(h, length: int, hop: int) -> int:
    return _check(lib().mbr_separate_workspace_size(h, length, hop))


def mbr_separate(h, wave_ptr: int, length: int, hop: int, ws_ptr: int, out_ptr: int, stream_ptr: int = 0) -> None:
    _check(lib().mbr_separate(h, C.c_void_p(wave_ptr), length, hop, C.c_void_p(ws_ptr), C.c_void_p(out_ptr),
                              C.c_void_p(stream_ptr)))


def mbr_separate_workspace_size_strided(h, length: int, hop: int, stride: int) -> int:
    return _check(lib().mbr_separate_workspace_size_strided(h, length, hop, stride))


def mbr_separate_strided(h, wave_ptr: int, length: int, hop: int, stride: int, ws_ptr: int, out_ptr: int,
                         stream_ptr: int = 0) -> None:
    _check(lib().mbr_separate_strided(h, C.c_void_p(wave_ptr), length, hop, stride, C.c_void_p(ws_ptr),
                                      C.c_void_p(out_ptr), C.c_void_p(stream_ptr)))


def stft(wave, n_fft: int, hop: int, stream=None):
    """wave: float32 CUDA tensor [channels, length] -> stft_repr [1, F*channels, T, 2]."""
    torch = _torch()
    _check_dense(wave)
    S, L = wave.shape
    out = torch.empty((1, (n_fft // 2 + 1) * S, 1 + L // hop, 2), dtype=torch.float32, device=wave.device)
    mbr_stft(wave.data_ptr(), S, L, n_fft, hop, out.data_ptr(), _stream_ptr(stream))
    return out


def istft_masked(spec, masks, channels: int, length: int, n_fft: int, hop: int, stream=None):
    """spec [1, F*S, T, 2] times masks [stems, F*S, T, 2] -> waves [stems, S, length]."""
    torch = _torch()
    _check_dense(spec)
    _check_dense(masks)
    stems, T = masks.shape[0], spec.shape[2]
    ws = torch.empty(mbr_istft_workspace_size(channels, n_fft, T, stems), dtype=torch.uint8, device=spec.device)
    out = torch.empty((stems, channels, length), dtype=torch.float32, device=spec.device)
    mbr_istft_masked(spec.data_ptr(), masks.data_ptr(), stems, channels, length, n_fft, hop, ws.data_ptr(),
                     out.data_ptr(), _stream_ptr(stream))
    _keep_for_stream(ws, stream)
    return out


def mbr_k_gemm_variants() -> int:
    return lib().mbr_k_gemm_variants()


# ----------------------------------------------------------------------------- marshalling helpers

def inventory(cfg: MbrConfig) -> List[Tuple[str, Tuple[int, ...], int]]:
    """The library's weight list as (index name, shape, kind) for the seeded weight generator."""
    n = mbr_core_weight_count(cfg)
    out = []
    for i in range(n):
        shape, kind = mbr_core_weight_info(cfg, i)
        out.append((f"w{i}", shape, kind))
    return out


def _torch():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible: the core runs only on an MI355X (gfx950)")
    return torch


def _check_dense(t) -> None:
    """The C ABI takes raw pointers to dense row-major float32 device arrays."""
    torch = _torch()
    if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()):
        raise ValueError("expected a contiguous float32 CUDA tensor")


def _stream_ptr(stream) -> int:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return int(getattr(stream, "cuda_stream", stream))


def _keep_for_stream(buf, stream) -> None:
    """A workspace allocated here (on torch's current stream) but used by work enqueued on
    `stream`: tell torch's caching allocator that `stream` uses it, so the block is not handed to
    another tensor before that stream has passed the work."""
    if stream is None:
        return
    torch = _torch()
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    if s.cuda_stream != torch.cuda.current_stream().cuda_stream:
        buf.record_stream(s)


class Core:
    """An mbr_core handle with its weights uploaded through torch device memory.

    weights: fp64 arrays holding values representable in cfg.dtype (e.g. from synth.draw_weights).
    """

    def __init__(self, cfg: MbrConfig, weights: Sequence[np.ndarray]):
        torch = _torch()
        self.cfg = cfg
        dev = []
        for w in weights:
            a = synth.storage_bytes(w, cfg.dtype)
            t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")
            dev.append(t)
        torch.cuda.synchronize()
        self.handle = mbr_core_create(cfg, [t.data_ptr() for t in dev])
        del dev
        self.S = cfg.audio_channels
        self.F = cfg.n_fft // 2 + 1

    def output_shape(self, batch: int) -> Tuple[int, ...]:
        T, S, F, st = self.cfg.frames, self.S, self.F, self.cfg.num_stems
        lead = (batch,) if st == 1 else (batch, st)
        if self.cfg.io_layout == synth.IO_FS_T_C:
            return lead + (F * S, T, 2)
        return lead + (S * 2, F, T)

    def forward(self, x, out=None, stream=None):
        """x: float32 CUDA tensor in the io layout; returns the masks tensor (asynchronous)."""
        torch = _torch()
        assert x.is_cuda and x.dtype == torch.float32 and x.is_contiguous()
        batch = x.shape[0]
        if out is None:
            out = torch.empty(self.output_shape(batch), dtype=torch.float32, device=x.device)
        mbr_core_forward(self.handle, x.data_ptr(), out.data_ptr(), batch, _stream_ptr(stream))
        return out

    def debug(self, x, stage: int, stream=None):
        torch = _torch()
        batch = x.shape[0]
        n = mbr_core_debug_size(self.handle, batch, stage)
        out = torch.empty(n, dtype=torch.float32, device=x.device)
        mbr_core_forward_debug(self.handle, x.data_ptr(), batch, stage, out.data_ptr(), _stream_ptr(stream))
        return out

    def separate(self, wave, hop: int, stream=None, stride: int = 0):
        """wave: float32 CUDA tensor [channels, length] -> stems [num_stems, channels, length].
        stride: chunk stride in samples (0: 0.9 chunk)."""
        torch = _torch()
        _check_dense(wave)
        S, L = wave.shape
        if S != self.S:
            raise ValueError(f"the core separates {self.S}-channel tracks, got {S} channels")
        ws = torch.empty(mbr_separate_workspace_size_strided(self.handle, L, hop, stride), dtype=torch.uint8,
                         device=wave.device)
        out = torch.empty((self.cfg.num_stems, S, L), dtype=torch.float32, device=wave.device)
        mbr_separate_strided(self.handle, wave.data_ptr(), L, hop, stride, ws.data_ptr(), out.data_ptr(),
                             _stream_ptr(stream))
        _keep_for_stream(ws, stream)
        return out

    def profile(self, x, out, stream=None):
        return mbr_core_forward_profiled(self.handle, x.data_ptr(), out.data_ptr(), x.shape[0], _stream_ptr(stream))

    def device_bytes(self) -> int:
        return mbr_core_device_bytes(self.handle)

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            mbr_core_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
