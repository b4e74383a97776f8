"""bench.py's argument checks, on the host (no GPU needed: they run before any device work)."""
import os
import subprocess
import sys

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)


def test_more_gpus_refused():
    p = run_bench("--gpus", "2")
    assert p.returncode != 0 and "one GPU" in p.stdout


def test_m_beyond_the_workloads_rows_refused():
    wl = workloads.WORKLOADS["nf4_g64_k4096_n14336"]
    p = run_bench("--workload", wl.name, "--m", str(wl.mmax + 1))
    assert p.returncode != 0 and f"between 1 and {wl.mmax}" in p.stdout


def test_m_zero_refused():
    p = run_bench("--workload", "int4_g64_k4096_n11008", "--m", "0")
    assert p.returncode != 0 and "between 1 and" in p.stdout
