"""Results do not depend on what the caller's workspace held before the call.

Every entry point is run twice on the same inputs, once with a zeroed workspace and once
with every byte 0xFF (each fp32 / bf16 value a NaN); the outputs must be bit-identical.
Shapes are chosen so that row blocks and vocabulary chunks are ragged (parts of the
gradient block and of the partial-sum arrays are never written in some launches).
"""
import numpy as np
import pytest
import torch

from chunked_lm_head_amd import synth

import gpu_util as gu

pytestmark = pytest.mark.gpu


def _ws(n, dev, fill):
    return torch.full((n,), fill, dtype=torch.uint8, device=dev)


def _same(a, b):
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


def test_cross_entropy_ignores_workspace_contents():
    from chunked_lm_head_amd import flce

    w = synth.custom("ws_ce", T=700, H=136, V=3001, chunk_rows=64, ignore_frac=0.05, seed=41)
    x = synth.make_inputs(w)
    dev = gu.device()
    h, W = gu.bf16_tensor(x.hidden, dev), gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    n = flce.workspace_bytes(w.T, w.H, w.V, w.chunk_rows)
    outs = []
    for fill in (0, 255):
        ws = _ws(n, dev, fill)
        out, lse, mean = flce.forward(h, W, y, chunk_rows=w.chunk_rows, workspace=ws)
        dh, dw = flce.backward(h, W, y, lse, chunk_rows=w.chunk_rows, workspace=ws,
                               grad_mean=torch.ones((), device=dev))
        torch.cuda.synchronize()
        outs.append((out, lse, mean, dh, dw))
    _same(*outs)
    assert bool(torch.isfinite(outs[0][4]).all())


def test_distillation_ignores_workspace_contents():
    from chunked_lm_head_amd import flce

    w = synth.distill_custom("ws_dst", T=700, Hs=136, Ht=200, V=3001, chunk_rows=64,
                             ignore_frac=0.05, seed=43)
    x = synth.make_distill_inputs(w)
    dev = gu.device()
    sh, sw = gu.bf16_tensor(x.s_hidden, dev), gu.bf16_tensor(x.s_weight, dev)
    th, tw = gu.bf16_tensor(x.t_hidden, dev), gu.bf16_tensor(x.t_weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    n = flce.distill_workspace_bytes(w.T, w.Hs, w.Ht, w.V, w.chunk_rows)
    outs = []
    for fill in (0, 255):
        r = flce.distill(sh, sw, th, tw, y, chunk_rows=w.chunk_rows, workspace=_ws(n, dev, fill),
                         grad_mean=torch.ones((), device=dev))
        torch.cuda.synchronize()
        outs.append(r)
    _same(*outs)
    assert bool(torch.isfinite(outs[0][3]).all())


@pytest.mark.parametrize("kind", ["grpo", "dpo", "kto"])
def test_policy_losses_ignore_workspace_contents(kind):
    from chunked_lm_head_amd import flce

    w = synth.policy_custom("ws_pol", 4, 175, 25, 136, 3001, chunk_rows=64, seed=47)
    x = synth.make_policy_inputs(w)
    dev = gu.device()
    h, W = gu.bf16_tensor(x.hidden, dev), gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    n = flce.policy_workspace_bytes(w.T, w.H, w.V, w.chunk_rows, w.n_seq)
    seq = torch.from_numpy(-1200.0 + 5.0 * x.seq_noise).to(dev)  # near pi_b: margins of order 1
    outs = []
    for fill in (0, 255):
        kw = dict(chunk_rows=w.chunk_rows, workspace=_ws(n, dev, fill),
                  grad_loss=torch.ones((), device=dev))
        if kind == "grpo":
            r = flce.grpo_loss(h, W, y, w.n_seq, torch.from_numpy(x.advantages).to(dev),
                               ref_logp=torch.from_numpy(-5.0 + x.ref_noise).to(dev), beta=0.1,
                               **kw)
        elif kind == "dpo":
            r = flce.dpo_loss(h, W, y, w.n_seq, seq, beta=0.1, **kw)
        else:
            r = flce.kto_loss(h, W, y, w.n_seq, seq, torch.from_numpy(x.desirable).to(dev),
                              beta=0.1, **kw)
        torch.cuda.synchronize()
        outs.append(r)
    _same(*outs)
    assert bool(torch.isfinite(outs[0][0]).all()) and bool(torch.isfinite(outs[0][3]).all())
