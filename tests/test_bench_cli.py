"""The benchmark's command-line contract, on the CPU: one GPU only, and the workloads it
offers (the measured ones, the calibration probes and the vendor reference points)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_workloads_offered():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("decode", "prefill", "moe_cont", "moe_mask", "moe_swiglu", "quant", "small",
              "hbm_ceiling", "vendor_prefill", "vendor_decode", "overlap_probe"):
        assert w in r.stdout, w
