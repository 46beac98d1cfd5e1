"""bench.py's command-line contract that needs no GPU: more than one GPU is refused with a
message (the benchmark measures one GPU), and the argument parser knows every mode."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = run_bench(env_extra={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "WORLD_SIZE 4" in r.stderr


def test_help_lists_the_modes():
    r = run_bench("--help")
    assert r.returncode == 0
    for mode in ("bench", "pmc-prefill", "pmc-copy", "segmented", "ablation", "pmc-ablation",
                 "pmc-mfma", "pmc-decode"):
        assert mode in r.stdout
    assert "--core-only" in r.stdout
