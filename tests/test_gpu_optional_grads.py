"""Either gradient output of the backward may be skipped (a frozen lm_head, or hidden
states that need no gradient); what is computed is bit-identical to the full call."""
import numpy as np
import pytest
import torch

from chunked_lm_head_amd import synth

import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case():
    w = synth.custom("optional_grads", T=700, H=264, V=3100, chunk_rows=32, ignore_frac=0.05,
                     seed=71)
    return synth.make_inputs(w)


def test_backward_skips_either_gradient():
    from chunked_lm_head_amd import flce

    x = _case()
    dev = gu.device()
    h, W = gu.bf16_tensor(x.hidden, dev), gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    cr = x.workload.chunk_rows
    _, lse, _ = flce.forward(h, W, y, chunk_rows=cr)
    g = torch.tensor(1.7, dtype=torch.float32, device=dev)
    dh, dw = flce.backward(h, W, y, lse, grad_mean=g, chunk_rows=cr)
    dh_only, none_w = flce.backward(h, W, y, lse, grad_mean=g, chunk_rows=cr, need_weight=False)
    none_h, dw_only = flce.backward(h, W, y, lse, grad_mean=g, chunk_rows=cr, need_hidden=False)
    torch.cuda.synchronize()
    assert none_w is None and none_h is None
    assert torch.equal(dh_only, dh)
    assert torch.equal(dw_only, dw)
    with pytest.raises(ValueError):
        flce.backward(h, W, y, lse, grad_mean=g, chunk_rows=cr, need_hidden=False,
                      need_weight=False)


def test_frozen_lm_head_through_autograd():
    from chunked_lm_head_amd import flce

    x = _case()
    dev = gu.device()
    y = torch.from_numpy(x.labels).to(dev)
    cr = x.workload.chunk_rows
    a = gu.bf16_tensor(x.hidden, dev).requires_grad_()
    b = gu.bf16_tensor(x.weight, dev).requires_grad_()
    (flce.chunked_linear_cross_entropy(a, b, y, chunk_rows=cr) * 3.0).backward()
    a2 = gu.bf16_tensor(x.hidden, dev).requires_grad_()
    b2 = gu.bf16_tensor(x.weight, dev)          # frozen
    (flce.chunked_linear_cross_entropy(a2, b2, y, chunk_rows=cr) * 3.0).backward()
    a3 = gu.bf16_tensor(x.hidden, dev)          # no gradient for the hidden states
    b3 = gu.bf16_tensor(x.weight, dev).requires_grad_()
    (flce.chunked_linear_cross_entropy(a3, b3, y, chunk_rows=cr) * 3.0).backward()
    torch.cuda.synchronize()
    assert b2.grad is None and a3.grad is None
    assert torch.equal(a2.grad, a.grad)
    assert torch.equal(b3.grad, b.grad)


def test_distill_and_policy_skip_either_gradient():
    from chunked_lm_head_amd import flce

    dev = gu.device()
    w = synth.distill_custom("optional_distill", T=300, Hs=128, Ht=192, V=1500, ws_std=0.3,
                             wt_std=0.3, ignore_frac=0.1, reduction="mean", seed=72)
    x = synth.make_distill_inputs(w)
    sh, sw = gu.bf16_tensor(x.s_hidden, dev), gu.bf16_tensor(x.s_weight, dev)
    th, tw = gu.bf16_tensor(x.t_hidden, dev), gu.bf16_tensor(x.t_weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    one = torch.ones((), dtype=torch.float32, device=dev)
    for div in ("kl", "jsd"):
        kw = dict(chunk_rows=w.chunk_rows, grad_mean=one, divergence=div, beta=0.4)
        _, _, dh, dw = flce.distill(sh, sw, th, tw, y, **kw)
        _, _, dh1, dw1 = flce.distill(sh, sw, th, tw, y, need_weight=False, **kw)
        _, _, dh2, dw2 = flce.distill(sh, sw, th, tw, y, need_hidden=False, **kw)
        torch.cuda.synchronize()
        assert dw1 is None and dh2 is None
        assert torch.equal(dh1, dh) and torch.equal(dw2, dw)

    pw = synth.custom("optional_policy", T=512, H=128, V=1200, chunk_rows=64, mode="logprob",
                      reduction="none", seq_len=128, prompt_len=16, seed=73)
    px = synth.make_inputs(pw)
    h, W = gu.bf16_tensor(px.hidden, dev), gu.bf16_tensor(px.weight, dev)
    py = torch.from_numpy(px.labels).to(dev)
    adv = torch.linspace(-1.0, 1.0, 4, dtype=torch.float32, device=dev)
    kw = dict(chunk_rows=64, beta=0.0, grad_loss=torch.tensor(0.8, device=dev))
    _, _, dh, dw = flce.grpo_loss(h, W, py, 4, adv, **kw)
    _, _, dh1, dw1 = flce.grpo_loss(h, W, py, 4, adv, need_weight=False, **kw)
    _, _, dh2, dw2 = flce.grpo_loss(h, W, py, 4, adv, need_hidden=False, **kw)
    torch.cuda.synchronize()
    assert dw1 is None and dh2 is None
    assert torch.equal(dh1, dh) and torch.equal(dw2, dw)
