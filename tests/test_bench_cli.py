"""bench.py's command line on a machine without a GPU: it measures one GPU
only, so --gpus above 1 stops with a message (exit status 2) before touching
a device, and --help lists the flags the timing contract uses."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _bench("--gpus", n)
        assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
        assert "one GPU" in (r.stdout + r.stderr)


def test_help_lists_the_timing_flags():
    r = _bench("--help")
    assert r.returncode == 0, r.stderr
    for flag in ("--gpus", "--steps", "--warmup", "--workload"):
        assert flag in r.stdout
