"""bench.py on the CPU: it compiles, refuses more than one GPU with a message, and prints its options."""
import os
import py_compile
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_bench_compiles():
    py_compile.compile(BENCH, doraise=True)


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "single GPU" in r.stdout + r.stderr, r.stdout + r.stderr


def test_bench_help():
    r = subprocess.run([sys.executable, BENCH, "--help"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0 and "--workload" in r.stdout
