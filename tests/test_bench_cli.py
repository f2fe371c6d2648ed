"""bench.py's command line without a GPU: it refuses more than one GPU with a
message and exit status 2 (the library has no multi-GPU path), and its options
parse."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, timeout=120)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _run("--gpus", n)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr
        assert r.stdout == ""  # no JSON line


def test_options_parse():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--granularity", "--pv", "--qk-bits", "--no-cpu",
                "--no-contrast", "--prep-flush", "--decode", "--copy-probe"):
        assert opt in r.stdout, opt
