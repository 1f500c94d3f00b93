"""The seeded input generator (CPU only)."""
import numpy as np
import torch

from chunked_lm_head_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0,
                                  65504.0, 1e-40, 3.0e38], dtype=np.float32)])
    ours = synth.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_workload_recipe():
    w = synth.WORKLOADS["tiny"]
    x = synth.make_inputs(w)
    assert x.hidden.shape == (67, 128) and x.hidden.dtype == np.uint16
    assert x.weight.shape == (1000, 128)
    assert (x.labels == synth.IGNORE_INDEX).sum() == 7          # round(0.10 * 67)
    used = x.labels[x.labels != synth.IGNORE_INDEX]
    assert used.min() >= 0 and used.max() < 1000
    assert x.grad_out is None
    assert synth.WORKLOADS["qwen3_8b_sft"].ignore_count == 819   # round(0.05 * 16384)
    # W ~ N(0, 1/H)
    wf = (x.weight.astype(np.uint32) << 16).view(np.float32)
    assert abs(wf.std() * np.sqrt(128) - 1.0) < 0.02


def test_deterministic_and_block_seeded():
    w = synth.custom("d", T=5000, H=16, V=300, seed=3)
    a = synth.make_inputs(w)
    b = synth.make_inputs(w)
    assert np.array_equal(a.hidden, b.hidden) and np.array_equal(a.weight, b.weight)
    assert np.array_equal(a.labels, b.labels)
    # the weight does not depend on T
    w2 = synth.custom("d", T=7, H=16, V=300, seed=3)
    assert np.array_equal(synth.make_inputs(w2).weight, a.weight)


def test_grpo_prompt_zeros():
    w = synth.custom("g", T=64, H=8, V=50, mode="logprob", reduction="none",
                     seq_len=16, prompt_len=4)
    x = synth.make_inputs(w)
    pos = np.arange(64) % 16
    assert np.all(x.grad_out[pos < 4] == 0.0)
    assert np.all(x.grad_out[pos >= 4] != 0.0)
