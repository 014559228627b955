"""Host-side logic of bench.py that runs without a GPU: parsing of the
amd-smi clock/power query, its skip under a profiler, and the refusal of
more than one GPU."""

import importlib.util
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture()
def bench(monkeypatch):
    for key in list(os.environ):
        if key.startswith("ROCPROF"):
            monkeypatch.delenv(key)
    monkeypatch.setenv("LD_PRELOAD", "")
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _fake_smi(payload):
    def run(cmd, capture_output, text, timeout):
        assert cmd[0] == "amd-smi" and "metric" in cmd
        return types.SimpleNamespace(stdout=json.dumps(payload), stderr="", returncode=0)
    return run


def _gpu(clocks, power):
    clock = {f"gfx_{i}": {"clk": {"value": c, "unit": "MHz"}} for i, c in enumerate(clocks)}
    clock["socclk_0"] = {"clk": {"value": 43, "unit": "MHz"}}
    return {"gpu": 0, "power": {"socket_power": {"value": power, "unit": "W"}}, "clock": clock}


def test_parses_gfx_clocks_and_power(bench, monkeypatch):
    monkeypatch.setattr(subprocess, "run", _fake_smi([_gpu([1800, 1700, 1900, 1800], 1390)]))
    r = bench.sample_clock_power()
    assert r == {"socket_power_w": 1390, "gfx_clock_mhz_mean": 1800.0, "gfx_clock_mhz_min": 1700.0,
                 "gfx_clock_mhz_max": 1900.0}


def test_accepts_the_gpu_data_wrapper(bench, monkeypatch):
    monkeypatch.setattr(subprocess, "run", _fake_smi({"gpu_data": [_gpu([2000, 2100], 1300)]}))
    r = bench.sample_clock_power()
    assert r["gfx_clock_mhz_mean"] == 2050.0 and r["socket_power_w"] == 1300


def test_unusable_output_gives_none(bench, monkeypatch):
    monkeypatch.setattr(subprocess, "run", _fake_smi({"unexpected": True}))
    assert bench.sample_clock_power() is None

    def missing(*a, **k):
        raise FileNotFoundError("amd-smi")
    monkeypatch.setattr(subprocess, "run", missing)
    assert bench.sample_clock_power() is None


def test_no_query_under_a_profiler_or_with_the_flag(bench, monkeypatch):
    def forbidden(*a, **k):
        raise AssertionError("amd-smi must not run here")
    monkeypatch.setattr(subprocess, "run", forbidden)
    monkeypatch.setenv("ROCPROF_KERNEL_TRACE", "1")
    assert bench.sample_clock_power() is None
    monkeypatch.delenv("ROCPROF_KERNEL_TRACE")
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/librocprofiler-sdk-tool.so")
    assert bench.sample_clock_power() is None
    monkeypatch.setenv("LD_PRELOAD", "")
    monkeypatch.setattr(bench, "_NO_CLOCK_SAMPLE", True)
    assert bench.sample_clock_power() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
