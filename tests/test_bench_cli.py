"""bench.py's command line runs its entry point: more than one GPU is refused
with a message (no GPU is touched), and the options parse."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    p = run("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_help_lists_the_modes():
    p = run("--help")
    assert p.returncode == 0
    for opt in ("--bwd", "--decode", "--gate", "--no-cpu-baseline"):
        assert opt in p.stdout


def test_unknown_workloads_are_refused_before_any_gpu_work():
    for args in (("--workload", "nope"), ("--also", "gqa32x8_t128k_b4096_k12_bf16,nope")):
        p = run(*args)
        assert p.returncode == 2
        assert "unknown workload nope" in p.stderr
