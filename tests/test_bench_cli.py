"""bench.py's command line on a host without a GPU (no GPU work is started)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT, env=e)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr and r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = run(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and r.stdout == ""


def test_no_gpu_fails_loudly_without_a_result_line():
    r = run("--steps", "1", "--warmup", "0", env={"HIP_VISIBLE_DEVICES": "", "CUDA_VISIBLE_DEVICES": ""})
    assert r.returncode != 0
    assert r.stdout.strip() == ""      # no JSON line: nothing was measured
    assert r.stderr.strip() != ""
