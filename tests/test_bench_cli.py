"""bench.py's command line on the CPU: it compiles, and asking for more than one GPU ends with a message and
exit status 2 before anything touches a device (the library has no multi-GPU path)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_bench_compiles():
    with open(BENCH) as f:
        compile(f.read(), BENCH, "exec")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_help_lists_the_warm_up_option():
    r = subprocess.run([sys.executable, BENCH, "--help"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "--warm-seconds" in r.stdout
