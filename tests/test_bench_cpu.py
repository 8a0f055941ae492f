"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the counter
figures' source-hash gate, and the roofline arithmetic of the JSON line."""
import importlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

bench = importlib.import_module("bench")


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_committed_counters_match_their_sources():
    # every entry is reported while its kernel sources are unchanged
    with open(bench.COUNTERS_FILE) as f:
        kernels = json.load(f)["kernels"]
    assert {"gemm_w1w3_swiglu", "attn_decode", "attn_prefill", "lm_head"} <= set(kernels)
    for name, entry in kernels.items():
        assert bench.measured_traffic(name) == pytest.approx(float(entry["bytes_per_launch"])), name
        # a bytes-per-launch figure is the fetched plus written KiB scaled by the copy calibration
        with open(bench.COUNTERS_FILE) as f:
            doc = json.load(f)
        scaled = (entry["fetch_kib"] * doc["fetch_factor"] + entry["write_kib"] * doc["write_factor"]) * 1024
        assert scaled == pytest.approx(entry["bytes_per_launch"], rel=1e-4), name


def test_counter_figures_are_dropped_when_a_source_changes(tmp_path, monkeypatch):
    with open(bench.COUNTERS_FILE) as f:
        doc = json.load(f)
    entry = doc["kernels"]["gemm_w1w3_swiglu"]
    src = tmp_path / "kernel.hip"
    src.write_text("// one version of the kernel\n")
    entry = dict(entry, sources=[os.path.relpath(src, ROOT)])
    import hashlib
    entry["sources_sha256"] = hashlib.sha256(src.read_bytes()).hexdigest()
    fake = tmp_path / "counters.json"
    fake.write_text(json.dumps({"kernels": {"k": entry}}))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(fake))
    assert bench.measured("k", "mfma_busy_pct") == pytest.approx(entry["mfma_busy_pct"])
    src.write_text("// the kernel edited after the counters were taken\n")
    assert bench.measured("k", "mfma_busy_pct") is None
    assert bench.measured_traffic("k") is None
    assert bench.measured("missing", "mfma_busy_pct") is None


def test_roofline_fractions_follow_work_over_time():
    kt = {"g": {"avg_ms": 1.5, "launches": 32, "ms_per_step": 48.0},
          "a": {"avg_ms": 0.2, "launches": 32, "ms_per_step": 6.4}}
    work = {"g": ("mfma", 1.924145348608e12), "a": ("hbm", 1.073741824e9), "absent": ("hbm", 1.0)}
    r = bench.kernel_rooflines(kt, work)
    assert set(r) == {"g", "a"}
    assert r["g"]["unit"] == "TFLOP/s" and r["a"]["unit"] == "GB/s"
    assert r["g"]["achieved"] == pytest.approx(1.924145348608e12 / 1.5e-3 / 1e12, abs=0.006)  # rounded to 0.01
    assert r["g"]["frac"] == pytest.approx(r["g"]["achieved"] / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    assert r["a"]["achieved"] == pytest.approx(1.073741824e9 / 0.2e-3 / 1e9, abs=0.006)
    assert r["a"]["frac"] == pytest.approx(r["a"]["achieved"] / bench.PEAK_HBM_GBS, abs=1e-4)
    assert bench.PEAK_BF16_TFLOPS == 2500.0 and bench.PEAK_HBM_GBS == 8000.0


def test_cpu_info_names_the_model_and_threads():
    info = bench.cpu_info()
    assert info["cores"] >= 1 and info["blas_threads"] >= 1
    assert isinstance(info["cpu"], str) and info["cpu"]
