"""The measurement script's refusals, which happen before any device work (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, env=env, timeout=300)


@pytest.mark.parametrize("args", [("--gpus", "2"), ("--gpus", "8", "--steps", "1")])
def test_more_than_one_gpu_is_refused(args):
    r = _bench(*args)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


@pytest.mark.parametrize("args, msg", [
    (("--token-shard", "3"), "does not split"),
    (("--workload", "grpo_logprob", "--token-shard", "8"), "does not split"),
    (("--workload", "distill_qwen3", "--token-shard", "2"), "cross-entropy workloads only"),
])
def test_bad_token_shards_are_refused(args, msg):
    r = _bench(*args)
    assert r.returncode != 0
    assert msg in r.stderr
