"""Host logic of bench.py and of the counter records it reads (no GPU needed): the one-GPU refusal,
the calibrated traffic arithmetic, the staleness check of a traffic record, and the committed bench
lines' own arithmetic against the FLOP model."""
import csv
import glob
import json
import os
import re
import subprocess
import sys

import pytest

from axial_band_split_amd import binding, profiling, roofline, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line for a configuration that was not measured


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for k, c, v in rows:
            wr.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_record_arithmetic(tmp_path):
    """Two instantiations of one kernel class count as one launch of both (the mean per dispatch of
    each, summed); other kernels are ignored; each counter is scaled by what it reads for a copy of
    known size."""
    a, b, other = "void mbr::block_kernel<A>(x)", "void mbr::block_reduce_kernel<A>(y)", "void mbr::attn_time2_kernel<A>(z)"
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, [(a, "FETCH_SIZE", 1000), (a, "FETCH_SIZE", 3000), (b, "FETCH_SIZE", 10),
                         (other, "FETCH_SIZE", 1e9), (a, "WRITE_SIZE", 1e9)])
    _counter_csv(write, [(a, "WRITE_SIZE", 400), (b, "WRITE_SIZE", 6), (b, "WRITE_SIZE", 2),
                         (other, "WRITE_SIZE", 1e9)])
    cal_f = tmp_path / "cal_fetch.csv"
    cal_w = tmp_path / "cal_write.csv"
    # the copy reads twice and writes once what it moves (in KiB): factors 1/2 and 1
    kib = profiling.CAL_BYTES / 1024
    _counter_csv(cal_f, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 2 * kib), (other, "FETCH_SIZE", 9 * kib)])
    _counter_csv(cal_w, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", kib)])
    rec = profiling.traffic_record(str(fetch), str(write), str(cal_f), str(cal_w), roofline.KIND_REGEX["block"],
                                   "cmd", sources=profiling.KIND_SOURCES["block"])
    assert rec["fetch_kib_per_dispatch"] == 2000 + 10
    assert rec["write_kib_per_dispatch"] == 400 + 4
    assert rec["fetch_factor"] == pytest.approx(0.5) and rec["write_factor"] == pytest.approx(1.0)
    assert rec["bytes_per_launch"] == pytest.approx((2010 * 0.5 + 404) * 1024)
    assert rec["source_sha"] == profiling.source_hash(profiling.KIND_SOURCES["block"])


def test_traffic_record_is_dropped_when_stale(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("wl", "block") is None                      # no record
    os.makedirs(tmp_path / "profiles")
    files = list(profiling.KIND_SOURCES["block"])
    rec = {"kernel_regex": roofline.KIND_REGEX["block"], "source_files": files,
           "source_sha": profiling.source_hash(files), "bytes_per_launch": 123.0}
    path = tmp_path / "profiles" / "traffic_wl.json"
    path.write_text(json.dumps(rec))
    assert bench.traffic_for("wl", "block") == 123.0
    assert bench.traffic_for("wl", "qkv") is None                        # another kernel class
    path.write_text(json.dumps(dict(rec, source_sha="0" * 16)))
    assert bench.traffic_for("wl", "block") is None                      # sources changed since
    path.write_text(json.dumps(dict(rec, kernel_regex="block_kernel")))
    assert bench.traffic_for("wl", "block") is None                      # other kernels counted


def test_source_hash_covers_only_the_named_files():
    files = profiling.KIND_SOURCES["block"]
    assert profiling.source_hash(files) == profiling.source_hash(tuple(reversed(files)))
    assert profiling.source_hash(files) != profiling.source_hash(files[:-1])
    assert profiling.source_hash(files) != profiling.source_hash()


RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "bench_*.json")))


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_committed_bench_lines_are_self_consistent(path):
    """Each committed bench line: the contract's fields, the throughput from its own step time, the
    dominant kernel's FLOP count from the FLOP model at that workload, its rate and fraction of the
    peak from its own launch time, and its traffic equal to the committed counter record's."""
    line = json.loads(open(path).read().strip().splitlines()[-1])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["higher_is_better"] is True and line["data"] == "synthetic"
    w = synth.WORKLOADS[line["config"]["workload"]]
    assert line["dtype"] == synth.DTYPE_NAMES[w.dtype]
    assert line["config"]["audio_seconds_per_step"] == pytest.approx(w.audio_seconds)
    assert line["value"] == pytest.approx(w.audio_seconds / (line["ms_per_step"] * 1e-3), rel=1e-9)

    roof = line["roofline"]
    kind = roof["kernel"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    assert roof["peak"] == roofline.PEAK_MFMA_TFLOPS[w.dtype]
    _, total_width, _ = binding.mbr_core_table_sizes(binding.config(w))
    s = roofline.shape_of(w, total_width)
    assert roof["flops_per_launch"] == pytest.approx(bench.kind_flops(s, kind, w), rel=1e-12)
    assert roof["avg_launch_ms"] == line["kernels"][kind]["avg_launch_ms"]
    assert roof["achieved"] == pytest.approx(roof["flops_per_launch"] / (roof["avg_launch_ms"] * 1e-3) / 1e12, rel=1e-9)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-12)
    assert kind == max(line["kernels"], key=lambda k: line["kernels"][k]["ms_per_step"])
    if roof["traffic"] is not None:
        rec = json.load(open(os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")))
        assert rec["kernel_regex"] == roofline.KIND_REGEX[kind]
        # a line may predate a re-take of the record on the same sources: two takes of the
        # counters differ by about 1e-5
        assert roof["traffic"] == pytest.approx(rec["bytes_per_launch"], rel=1e-3)

    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == line["unit"] and cpu["cores"] >= 1 and cpu["sample"]


TRAFFIC = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))


@pytest.mark.parametrize("path", TRAFFIC, ids=[os.path.basename(p) for p in TRAFFIC])
def test_committed_traffic_records_are_self_consistent(path):
    """A traffic record's bytes follow from its own counter means and calibration factors, the
    factors from the calibration copy it names, and its command runs files of this repository."""
    rec = json.load(open(path))
    want = (rec["fetch_kib_per_dispatch"] * rec["fetch_factor"] + rec["write_kib_per_dispatch"] * rec["write_factor"]) * 1024
    assert rec["bytes_per_launch"] == pytest.approx(want, rel=1e-12)
    m = re.match(r"device copy of (\d+) bytes: FETCH_SIZE (\d+) KiB, WRITE_SIZE (\d+) KiB", rec["calibration"])
    assert m, rec["calibration"]
    moved, f_kib, w_kib = (int(g) for g in m.groups())
    assert moved == profiling.CAL_BYTES
    # the calibration line prints whole KiB (about 4e-6 of the copy's counter reading)
    assert rec["fetch_factor"] == pytest.approx(moved / (f_kib * 1024), rel=1e-5)
    assert rec["write_factor"] == pytest.approx(moved / (w_kib * 1024), rel=1e-5)
    assert rec["kernel_regex"] in roofline.KIND_REGEX.values()
    assert rec["source_files"] and all(os.path.exists(os.path.join(ROOT, "axial_band_split_amd", "csrc", f))
                                       for f in rec["source_files"])
    for f in re.findall(r"\$R/(\S+\.py)", rec["command"]):
        assert os.path.exists(os.path.join(ROOT, f)), f


SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))


@pytest.mark.parametrize("path", SUMMARIES, ids=[os.path.basename(p) for p in SUMMARIES])
def test_profile_summaries_name_a_command_of_committed_files(path):
    """Every rocprofv3 summary is short text that gives the command it came from, and that command
    runs files of this repository."""
    text = open(path).read()
    assert len(text) < 16 * 1024
    cmd = re.search(r"^Command[^:]*: (.+)$", text, re.M)
    assert cmd, "no command line"
    scripts = re.findall(r"python3 (?:\$R/)?(\S+?\.py)\b", cmd.group(1))   # $R or relative to the root
    assert scripts, cmd.group(1)
    for f in scripts:
        assert os.path.exists(os.path.join(ROOT, f)), f


@pytest.mark.parametrize("path", TRAFFIC, ids=[os.path.basename(p) for p in TRAFFIC])
def test_algorithmic_bytes_do_not_exceed_the_measured_traffic(path):
    """The byte model counts every operand once, so a launch cannot move fewer HBM bytes than it
    gives; a term counted twice or in the wrong width would show here as more than was measured."""
    rec = json.load(open(path))
    name = os.path.basename(path)[len("traffic_"):-len(".json")]
    w = synth.WORKLOADS[name]
    kind = next(k for k, v in roofline.KIND_REGEX.items() if v == rec["kernel_regex"])
    _, total_width, _ = binding.mbr_core_table_sizes(binding.config(w))
    algo = roofline.bytes_per_launch(roofline.shape_of(w, total_width))[kind]
    assert 0.5 * rec["bytes_per_launch"] < algo <= rec["bytes_per_launch"]


def test_sweep_rows_follow_from_their_step_times():
    """Each row of the committed sweep: audio seconds per step = B * T * hop / sample rate (hop 441
    at 44.1 kHz, whatever the stem count), divided by the row's step time."""
    rows = [ln.split("|")[1:-1] for ln in open(os.path.join(ROOT, "profiles", "sweep_chunk11s_fp16.md"))
            if ln.startswith("| ") and not ln.startswith("| workload")]
    assert len(rows) >= 8
    for r in rows:
        B, T, ms, rate = int(r[1]), int(r[2]), float(r[4]), float(r[5])
        assert rate == pytest.approx(B * T * 441 / 44100 / (ms * 1e-3), rel=2e-3), r[0]


def _ignored(path: str, pattern: str) -> bool:
    """tar-style exclusion: './p' anchors at the top, any other pattern matches at any depth."""
    import fnmatch
    parts = path.split("/")
    if pattern.startswith("./"):
        p = pattern[2:]
        return any(fnmatch.fnmatch("/".join(parts[:i]), p) for i in range(1, len(parts) + 1))
    return any(fnmatch.fnmatch("/".join(parts[i:j]), pattern)
               for i in range(len(parts)) for j in range(i + 1, len(parts) + 1))


def test_gpu_runs_receive_every_file_they_load():
    """No pattern of the push's ignore list drops the library's sources, the oracle, the header,
    the bench and its counter records, or a test that the GPU suite collects."""
    ign = os.path.join(ROOT, ".gpurunignore")
    patterns = [ln.strip() for ln in open(ign) if ln.strip() and not ln.startswith("#")]
    files = subprocess.run(["git", "ls-files"], cwd=ROOT, capture_output=True, text=True).stdout.split()
    if not files:
        pytest.skip("not a git checkout")
    host_only = {"tests/test_host_sanitized.py", "tests/host_tables_driver.cpp"}
    needed = [f for f in files if f.split("/")[0] in ("axial_band_split_amd", "oracle", "include", "profiles", "tests")
              or f in ("bench.py", "__graft_entry__.py")]
    needed = [f for f in needed if f not in host_only and not f.endswith(".md")]
    assert "profiles/traffic_chunk11s_fp16.json" in needed
    for f in needed:
        hit = [p for p in patterns if _ignored(f, p)]
        assert not hit, (f, hit)
    for f in host_only:
        assert any(_ignored(f, p) for p in patterns), f
