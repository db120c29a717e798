"""The measurement script's command line, on the CPU (no GPU is touched):
it refuses more than one GPU with a message, and its workload table names the
shapes the parity tests and the profiles use."""
import os
import subprocess
import sys

import esg_inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_help_lists_the_modes():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--workload", "--steps", "--warmup", "--backward-streams", "--k-sweep", "--skew", "--inference"):
        assert flag in r.stdout


def test_default_workload_is_the_largest_sparse_shape():
    # the 1.3B shape at 32768 tokens, k = 11 of 43 groups of 128
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--workload", default="s1p3b_bf16")' in src
    w = I.WORKLOADS["s1p3b_bf16"]
    assert (w.tokens, w.d_model, w.d_ff, w.group_size, w.k) == (32768, 2048, 5504, 128, 11)
    sparse = [v for v in I.WORKLOADS.values() if not getattr(v, "dense", False) and v.dtype == "bf16"]
    assert max(v.tokens * v.k * v.group_size * v.d_model for v in sparse) == \
        w.tokens * w.k * w.group_size * w.d_model
