"""Host-side checks of libmbr_core.so (no GPU needed): exports, tables, inventory, config errors."""
import os
import re
import subprocess

import numpy as np
import pytest

from axial_band_split_amd import binding, synth
from oracle import model as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mbr_core.h")


def _oracle_cfg(w: synth.Workload, **kw) -> M.CoreConfig:
    d = dict(sample_rate=w.sample_rate, n_fft=w.n_fft, audio_channels=w.audio_channels, num_bands=w.num_bands,
             dim=w.dim, depth=w.depth, heads=w.heads, dim_head=w.dim_head, ff_mult=w.ff_mult,
             mask_hidden_mult=w.mask_hidden_mult, mask_depth=w.mask_depth, num_stems=w.num_stems)
    d.update(kw)
    return M.CoreConfig(**d)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mbr_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    binding.lib()
    declared = _declared_functions()
    assert declared == sorted(binding.SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (mbr_\w+)", out))
    assert set(declared) <= exported


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_tables_bit_exact_with_oracle(name):
    w = synth.WORKLOADS[name]
    cfg = binding.config(w)
    got = binding.mbr_core_tables(cfg)
    t = _oracle_cfg(w).tables()
    S = w.audio_channels
    assert got["band_bins"].tolist() == [len(b) for b in t.bins]
    assert got["band_offset"].tolist() == [0] + np.cumsum(t.widths).tolist()
    assert got["gather_pair"].tolist() == np.concatenate(t.pairs).tolist()
    assert got["bin_count"].tolist() == t.counts.tolist()
    # inverse index: the slots of every pair, ascending, -1 where one band covers the bin
    gp = np.concatenate(t.pairs)
    inv = np.full((t.n_freqs * S, 2), -1)
    for p in range(t.n_freqs * S):
        slots = np.nonzero(gp == p)[0]
        inv[p, :len(slots)] = slots
    assert np.array_equal(got["inv_slot"].reshape(-1, 2), inv)
    want_w = (1.0 / np.repeat(t.counts, S)).astype(np.float32)
    assert got["inv_weight"].tobytes() == want_w.tobytes()


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_inventory_matches_oracle(name):
    w = synth.WORKLOADS[name]
    lib_inv = binding.inventory(binding.config(w))
    ora_inv = M.inventory(_oracle_cfg(w))
    assert [s for _, s, _ in lib_inv] == [tuple(s) for _, s, _ in ora_inv]
    assert [k for _, _, k in lib_inv] == [k for _, _, k in ora_inv]


def test_inventory_with_two_stems_and_deeper_mask():
    w = synth.WORKLOADS["tiny_fp32"].replace(num_stems=2, mask_depth=3)
    lib_inv = binding.inventory(binding.config(w))
    ora_inv = M.inventory(_oracle_cfg(w))
    assert [s for _, s, _ in lib_inv] == [tuple(s) for _, s, _ in ora_inv]


def test_param_count_through_the_library():
    cfg = binding.config(synth.WORKLOADS["chunk11s_fp16"])
    total = sum(int(np.prod(s)) for _, s, _ in binding.inventory(cfg))
    assert total == 228202788


@pytest.mark.parametrize("field,value", [("dim", 100), ("dim_head", 48), ("dtype", 7), ("io_layout", 3),
                                         ("num_bands", 0), ("frames", 0), ("max_batch", 0), ("n_fft", 7)])
def test_invalid_configs_are_rejected(field, value):
    cfg = binding.config(synth.WORKLOADS["tiny_fp32"], **{field: value})
    with pytest.raises(binding.MbrError) as e:
        binding.mbr_core_weight_count(cfg)
    assert e.value.code == binding.MBR_E_CONFIG
    assert "invalid config" in binding.mbr_last_error()


def test_band_with_no_bin_is_a_config_error():
    """Too many bands for the bins: some triangle falls between two bins."""
    cfg = binding.config(synth.WORKLOADS["tiny_fp32"], n_fft=32, num_bands=40)
    with pytest.raises(binding.MbrError) as e:
        binding.mbr_core_table_sizes(cfg)
    assert e.value.code == binding.MBR_E_CONFIG


def test_weight_info_index_out_of_range():
    cfg = binding.config(synth.WORKLOADS["tiny_fp32"])
    n = binding.mbr_core_weight_count(cfg)
    with pytest.raises(binding.MbrError) as e:
        binding.mbr_core_weight_info(cfg, n)
    assert e.value.code == binding.MBR_E_ARG


SPLIT_62 = (4,) * 20 + (8,) * 16 + (16,) * 12 + (32,) * 8 + (62,) * 5 + (59,)


@pytest.mark.parametrize("zero_dc", [0, 1])
def test_explicit_band_table_and_zero_dc_bit_exact_with_oracle(zero_dc):
    w = synth.WORKLOADS["chunk11s_fp16"].replace(num_bands=62, band_bins=SPLIT_62, zero_dc=zero_dc)
    got = binding.mbr_core_tables(binding.config(w))
    t = _oracle_cfg(w, num_bands=62, band_bins=SPLIT_62, zero_dc=bool(zero_dc)).tables()
    assert got["band_bins"].tolist() == list(SPLIT_62)
    assert got["gather_pair"].tolist() == np.concatenate(t.pairs).tolist()
    assert got["bin_count"].tolist() == [1] * 1025
    inv = got["inv_slot"].reshape(-1, 2)
    assert inv[:, 1].tolist() == [-1] * (1025 * 2)
    assert inv[:, 0].tolist() == list(range(1025 * 2))
    want = np.ones(1025 * 2, dtype=np.float32)
    if zero_dc:
        want[:2] = 0.0
    assert got["inv_weight"].tobytes() == want.tobytes()
    lib_inv = binding.inventory(binding.config(w))
    ora_inv = M.inventory(_oracle_cfg(w, num_bands=62, band_bins=SPLIT_62))
    assert [s for _, s, _ in lib_inv] == [tuple(s) for _, s, _ in ora_inv]


@pytest.mark.parametrize("bins", [(500, 524), (0, 1025), (1025, 0), (600, 426)])
def test_bad_band_tables_are_refused(bins):
    w = synth.WORKLOADS["chunk11s_fp16"].replace(num_bands=2, band_bins=bins)
    with pytest.raises(binding.MbrError) as e:
        binding.mbr_core_weight_count(binding.config(w))
    assert e.value.code == -2


def test_header_is_plain_c_and_links(tmp_path):
    """A C99 program that includes the header, takes the address of every function it declares
    (so each must link) and calls the host queries: the boundary needs no C++ and no torch."""
    names = _declared_functions()
    w = synth.WORKLOADS["tiny_fp32"]
    src = ["#include <stdio.h>", "#include <string.h>", '#include "mbr_core.h"',
           "typedef void (*fn)(void);",
           "static const fn all[] = {" + ", ".join(f"(fn){n}" for n in names) + "};",
           "int main(void) {",
           "  mbr_config bad; memset(&bad, 0, sizeof bad);",
           "  int rc = mbr_core_weight_count(&bad);",
           "  const char* msg = mbr_last_error();",
           "  if (rc != MBR_E_CONFIG || strncmp(msg, \"invalid config\", 14) != 0) return 1;",
           "  mbr_config c; memset(&c, 0, sizeof c);",
           f"  c.sample_rate = {w.sample_rate}; c.n_fft = {w.n_fft}; c.audio_channels = {w.audio_channels};",
           f"  c.num_bands = {w.num_bands}; c.dim = {w.dim}; c.depth = {w.depth}; c.heads = {w.heads};",
           f"  c.dim_head = {w.dim_head}; c.ff_mult = {w.ff_mult}; c.mask_hidden_mult = {w.mask_hidden_mult};",
           f"  c.mask_depth = {w.mask_depth}; c.num_stems = {w.num_stems}; c.max_batch = 1; c.frames = {w.frames};",
           f"  c.dtype = {w.dtype}; c.io_layout = {w.io_layout}; c.band_bins = NULL;",
           "  int n = mbr_core_weight_count(&c);",
           "  if (n <= 0) return 2;",
           "  printf(\"%d %d\\n\", n, (int)(sizeof all / sizeof all[0]));",
           "  return 0;",
           "}"]
    (tmp_path / "abi.c").write_text("\n".join(src) + "\n")
    libdir = os.path.dirname(binding.LIB_PATH)
    exe = tmp_path / "abi"
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror=implicit-function-declaration",
                         "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.dirname(HEADER)}",
                         str(tmp_path / "abi.c"), "-o", str(exe), f"-L{libdir}", "-lmbr_core",
                         f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stderr)
    n, count = map(int, run.stdout.split())
    assert n == binding.mbr_core_weight_count(binding.config(w))
    assert count == len(names)
