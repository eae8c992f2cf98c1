"""bench.py entry point on the host: the command line parses, a multi-GPU
request is refused with a message, and the rocprof summary mode runs on an
empty directory."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_help():
    r = _run("--help")
    assert r.returncode == 0 and "--steps" in r.stdout


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_rocprof_summary_of_nothing(tmp_path):
    r = _run("--rocprof-summary", str(tmp_path))
    assert r.returncode == 0, r.stderr
    assert "traffic-json: {}" in r.stdout
