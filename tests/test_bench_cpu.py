"""Host-side pieces of bench.py: the one-GPU contract, the rocm-smi reader and
the traffic record's source check (no GPU needed)."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_smi_reader_parses_clock_and_power(monkeypatch):
    b = _bench()

    class Out:
        stdout = ('WARNING: low-power state\n\n'
                  + json.dumps({"card0": {"mclk clock speed:": "(2000Mhz)",
                                          "sclk clock level:": "S",
                                          "sclk clock speed:": "(2100Mhz)",
                                          "Current Socket Graphics Package Power (W)": "812.0"}}))
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: Out())
    assert b.smi_snapshot() == {"sclk_mhz": 2100.0, "power_w": 812.0}


def test_smi_reader_tolerates_a_missing_tool(monkeypatch):
    b = _bench()

    def boom(*a, **k):
        raise FileNotFoundError("rocm-smi")
    monkeypatch.setattr(subprocess, "run", boom)
    assert b.smi_snapshot() == {}


def test_stored_traffic_requires_matching_sources(tmp_path, monkeypatch):
    b = _bench()
    rec = {"kernel": "mfma_256x256", "workload": "S4096", "source_sha": b.kernel_source_sha(),
           "traffic_bytes": 123}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(f))
    assert b.stored_traffic("mfma_256x256", "S4096") == 123
    assert b.stored_traffic("mfma_128x128", "S4096") is None
    assert b.stored_traffic("mfma_256x256", "S2048") is None
    rec["source_sha"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert b.stored_traffic("mfma_256x256", "S4096") is None
