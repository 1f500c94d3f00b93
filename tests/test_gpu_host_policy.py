"""Integration options around the kernels, on the GPU: hidden states offloaded
to host memory between forward and backward, and hidden-state mini-batches
with the lm_head gradient accumulated across them (Unsloth GRPO page, sections
on hidden-state chunking and on offloading log-softmax activations)."""
import numpy as np
import pytest
import torch

from chunked_lm_head_amd import synth
from oracle import flce_oracle as o

import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case(T=780, D=256, V=3001, seed=31):
    w = synth.custom("hp", T=T, H=D, V=V, chunk_rows=64, w_std=0.3, ignore_frac=0.05,
                     mode="logprob", reduction="none", seed=seed, seq_len=260, prompt_len=40)
    return synth.make_inputs(w)


def test_offload_gives_identical_results():
    from chunked_lm_head_amd import flce

    x = _case()
    dev = gu.device()
    g = torch.from_numpy(x.grad_out).to(dev)
    y = torch.from_numpy(x.labels).to(dev)
    res = []
    for offload in (False, True):
        h = gu.bf16_tensor(x.hidden, dev).requires_grad_()
        W = gu.bf16_tensor(x.weight, dev).requires_grad_()
        lp = flce.selective_log_softmax(h, W, y, chunk_rows=64, temperature=0.9,
                                        offload=offload)
        (lp * g).sum().backward()
        torch.cuda.synchronize()
        res.append((lp.detach().cpu(), h.grad.cpu(), W.grad.cpu()))
    for a, b in zip(*res):
        assert torch.equal(a, b)
    f = o.forward(x.hidden, x.weight, x.labels, synth.IGNORE_INDEX, "logprob",
                  transform=o.LogitTransform(temperature=0.9))
    assert gu.max_abs(res[1][0].numpy(), f.out) <= gu.OUT_TOL


def test_offloaded_hidden_states_live_on_the_host():
    from chunked_lm_head_amd import flce

    x = _case(T=260)
    dev = gu.device()
    h = gu.bf16_tensor(x.hidden, dev).requires_grad_()
    W = gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    lp = flce.selective_log_softmax(h, W, y, chunk_rows=64, offload=True)
    node = lp.grad_fn
    assert node.hidden_host.device.type == "cpu" and node.hidden_host.is_pinned()
    assert all(t.data_ptr() != h.data_ptr() for t in node.saved_tensors)


@pytest.mark.parametrize("m", [1, 3])
def test_mini_batches_match_the_oracle(m):
    from chunked_lm_head_amd import flce

    x = _case()
    dev = gu.device()
    hfull = gu.bf16_tensor(x.hidden, dev)
    W = gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    g = torch.from_numpy(x.grad_out).to(dev)
    T = x.hidden.shape[0]
    bounds = [T * i // m for i in range(m + 1)]

    def hidden_fn(i, n):
        return hfull[bounds[i]:bounds[i + 1]].clone()   # a fresh mini-batch of hidden states

    logp, dh, dw = flce.mini_batched_log_softmax(hidden_fn, W, y, m, grad_out=g, chunk_rows=64)
    torch.cuda.synchronize()
    f = o.forward(x.hidden, x.weight, x.labels, synth.IGNORE_INDEX, "logprob")
    rdh, rdw = o.backward(x.hidden, x.weight, x.labels, synth.IGNORE_INDEX, "logprob",
                          grad_out=x.grad_out)
    assert gu.max_abs(logp.cpu().numpy(), f.out) <= gu.OUT_TOL
    assert gu.rel_fro(dh.float().cpu().numpy(), rdh) <= gu.GRAD_TOL
    assert gu.rel_fro(dw.cpu().numpy(), rdw) <= gu.GRAD_TOL


def test_auto_tune_reads_free_memory():
    from chunked_lm_head_amd import flce

    r = flce.auto_tune(4, 8192, 4096, 128000)
    free, _ = torch.cuda.mem_get_info()
    assert r["bytes_needed"] <= 0.9 * free
    assert r["mini_batches"] >= 1 and r["chunk_rows"] >= 1
