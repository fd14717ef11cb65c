"""The host-side table code (csrc/tables.cpp) built with g++ under the address and undefined-behaviour
sanitizers, run on every workload, an explicit 62-band table and refused tables: no sanitizer report,
and tables, inventory and rotary tables identical to those of the shipped library."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from axial_band_split_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "axial_band_split_amd", "csrc")
HIP_INC = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INC),
                                reason="needs g++ and the HIP headers")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("san") / "host_tables_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INC, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "tables.cpp"), os.path.join(ROOT, "tests", "host_tables_driver.cpp"),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return out


def _run(driver, w: synth.Workload):
    cfg = binding.config(w)
    fields = [cfg.sample_rate, cfg.n_fft, cfg.audio_channels, cfg.num_bands, cfg.dim, cfg.depth, cfg.heads,
              cfg.dim_head, cfg.ff_mult, cfg.mask_hidden_mult, cfg.mask_depth, cfg.num_stems, cfg.max_batch,
              cfg.frames, cfg.dtype, cfg.io_layout, cfg.zero_dc]
    bins = list(w.band_bins) if w.band_bins else []
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([driver] + [str(x) for x in fields + bins], capture_output=True, text=True, env=env)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
    out = {}
    for line in r.stdout.splitlines():
        k, *v = line.split()
        out.setdefault(k, []).append(v)
    return cfg, out


def _ints(out, key):
    return [int(x) for x in out[key][0]]


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_sanitized_tables_match_the_library(driver, name):
    w = synth.WORKLOADS[name]
    cfg, out = _run(driver, w)
    assert _ints(out, "rc") == [0]
    got = binding.mbr_core_tables(cfg)
    assert _ints(out, "band_bins") == got["band_bins"].tolist()
    assert _ints(out, "band_offset") == got["band_offset"].tolist()
    assert _ints(out, "gather_pair") == got["gather_pair"].tolist()
    assert _ints(out, "inv_slot") == got["inv_slot"].reshape(-1).tolist()
    assert _ints(out, "bin_count") == got["bin_count"].tolist()
    bits = np.array(_ints(out, "inv_weight_bits"), dtype=np.int64).astype(np.uint32)
    assert bits.tobytes() == got["inv_weight"].astype(np.float32).view(np.uint32).tobytes()
    shapes = _ints(out, "inventory")
    lib = [s for _, s, _ in binding.inventory(cfg)]
    assert [tuple(x for x in (shapes[2 * i], shapes[2 * i + 1])) for i in range(len(lib))] == \
        [(s[0], s[1] if len(s) > 1 else 1) for s in lib]
    ropes = out["rope"]
    assert [int(r[0]) for r in ropes] == [w.frames, 64]
    assert [int(r[1]) for r in ropes] == [w.frames * w.dim_head // 2, 64 * w.dim_head // 2]


def test_sanitized_explicit_band_table(driver):
    split = (4,) * 20 + (8,) * 16 + (16,) * 12 + (32,) * 8 + (62,) * 5 + (59,)
    w = synth.WORKLOADS["chunk11s_fp16"].replace(num_bands=62, band_bins=split, zero_dc=1)
    cfg, out = _run(driver, w)
    assert _ints(out, "rc") == [0]
    assert _ints(out, "band_bins") == list(split)
    assert _ints(out, "gather_pair") == binding.mbr_core_tables(cfg)["gather_pair"].tolist()


@pytest.mark.parametrize("bins", [(500, 524), (0, 1025), (1025, 0), (600, 426)])
def test_sanitized_refusals(driver, bins):
    w = synth.WORKLOADS["chunk11s_fp16"].replace(num_bands=2, band_bins=bins)
    _, out = _run(driver, w)
    assert _ints(out, "rc") == [-2]
