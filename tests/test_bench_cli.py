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


def _bench_module():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_backward_flops_count_the_tiles_that_run():
    """Executed backward FLOPs when token tiles without gradient are left out: counted here
    token by token (a token's tile runs if any token of its 256 has a gradient; the
    recompute, dH and dW all run exactly the tiles that run)."""
    import numpy as np

    bench = _bench_module()
    V, D = 1000, 64
    rng = np.random.default_rng(5)
    cases = [
        (np.ones(2600, bool), 2816),                               # all active
        (np.zeros(700, bool), 768),                                # nothing active
        (np.ones(2600, bool), 256),                                # one-tile row blocks
    ]
    a = np.ones(2600, bool)
    for t in (0, 1, 5, 10):                                        # holes incl. ragged tail
        a[t * 256:(t + 1) * 256] = False
    cases.append((a, 2816))
    b = rng.random(5000) < 0.002                                   # sparse: most tiles empty
    cases += [(b, 1024), (b, 4096)]
    for active, R in cases:
        T = active.shape[0]
        got = bench.backward_flops(active, R, V, D)
        tile_on = [active[(t // 256) * 256:(t // 256 + 1) * 256].any() for t in range(T)]
        gd = sum(tile_on)
        assert got["bwd_grad"] == got["bwd_dh"] == got["bwd_dw"] == 2.0 * V * D * gd
        assert got["token_tiles"] == -(-T // 256)
        if active.all():
            assert got["bwd_grad"] == 2.0 * T * V * D
    # the holes case by hand: tiles 2-4 and 6-9 run, 7 full tiles
    got = bench.backward_flops(a, 2816, V, D)
    assert got["bwd_grad"] == got["bwd_dw"] == 2.0 * V * D * 7 * 256
    assert got["skipped_token_tiles"] == 4
