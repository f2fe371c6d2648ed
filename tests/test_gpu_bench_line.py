"""bench.py's JSON line on the GPU: one run of the small self-attention
workload and one decode run, each printing exactly one line with the fields
the measurement reports (throughput, roofline with its bound and peak,
accuracy against float64, the 16-bit contrast)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def _line(*args):
    print("case bench.py " + " ".join(args), flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       cwd=ROOT, timeout=240)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-3000:]
    return json.loads(lines[0])


def _common(d, steps, warmup):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "accuracy"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["data"] == "synthetic" and "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] in ("mfma", "hbm") and r["peak"] > 0 and 0 < r["frac"] < 1
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    a = d["accuracy"]
    assert 0.99 < a["cos"] <= 1.0 and 0 <= a["rel_l1"] < 0.1 and a["rows"] > 0


def test_prefill_line():
    d = _line("--workload", "1", "--steps", "3", "--warmup", "1", "--no-cpu")
    _common(d, 3, 1)
    assert d["unit"] == "TOPS" and d["roofline"]["bound"] == "mfma" and d["roofline"]["unit"] == "TOPS"
    assert d["prep"]["ms_per_launch"] > 0 and 0 < d["prep"]["frac_hbm"] < 1
    assert d["config"]["workload"] == "selfattn_b1_h2_n256_d64_f16"
    for key in ("contrast", "contrast_naive"):
        assert "ms_per_call" in d[key] or "error" in d[key], d[key]


def test_decode_line():
    d = _line("--decode", "6", "--steps", "20", "--warmup", "2", "--no-cpu")
    _common(d, 20, 2)
    assert d["unit"] == "GB/s" and d["roofline"]["bound"] == "hbm"
    assert 0 < d["cache"]["ratio"] < 1
