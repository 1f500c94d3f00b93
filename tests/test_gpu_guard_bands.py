"""Nothing is written outside the outputs and the workspace: every buffer the library
writes is placed inside a larger allocation whose guard bands hold a byte pattern, and
after forward, backward, distillation and a policy call the bands are unchanged."""
import numpy as np
import pytest
import torch

from chunked_lm_head_amd import synth

import gpu_util as gu

pytestmark = pytest.mark.gpu

BAND = 8192          # guard bytes on each side (a multiple of 256, so the view stays aligned)
PATTERN = 0xA5


class Guarded:
    def __init__(self, shape, dtype, dev):
        nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.nbytes = nbytes
        self.raw = torch.full((nbytes + 2 * BAND,), PATTERN, dtype=torch.uint8, device=dev)
        self.t = self.raw[BAND:BAND + nbytes].view(dtype).view(shape)

    def intact(self):
        lo = self.raw[:BAND]
        hi = self.raw[BAND + self.nbytes:]
        return bool((lo == PATTERN).all()) and bool((hi == PATTERN).all())


def _inputs():
    w = synth.custom("guard", T=333, H=136, V=1500, chunk_rows=16, ignore_frac=0.1, seed=81)
    return w, synth.make_inputs(w)


def test_cross_entropy_writes_stay_inside_their_buffers():
    from chunked_lm_head_amd import flce

    w, x = _inputs()
    dev = gu.device()
    h, W = gu.bf16_tensor(x.hidden, dev), gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    T, D, V = w.T, w.H, w.V
    bufs = dict(out=Guarded((T,), torch.float32, dev), lse=Guarded((T,), torch.float32, dev),
                mean=Guarded((), torch.float32, dev), dh=Guarded((T, D), torch.bfloat16, dev),
                dw=Guarded((V, D), torch.float32, dev),
                ws=Guarded((flce.workspace_bytes(T, D, V, w.chunk_rows),), torch.uint8, dev))
    for mode, tr in (("nll", {}), ("logprob", dict(logit_softcapping=3.0, temperature=0.9))):
        flce.forward(h, W, y, chunk_rows=w.chunk_rows, mode=mode, transform=tr,
                     workspace=bufs["ws"].t, out=bufs["out"].t, lse=bufs["lse"].t,
                     mean=bufs["mean"].t)
        flce.backward(h, W, y, bufs["lse"].t, grad_mean=torch.ones((), device=dev),
                      chunk_rows=w.chunk_rows, mode=mode, transform=tr,
                      grad_hidden=bufs["dh"].t, grad_weight=bufs["dw"].t,
                      workspace=bufs["ws"].t)
        flce.backward(h, W, y, bufs["lse"].t, grad_mean=torch.ones((), device=dev),
                      chunk_rows=w.chunk_rows, mode=mode, transform=tr,
                      grad_weight=bufs["dw"].t, accumulate=True, workspace=bufs["ws"].t,
                      need_hidden=False)
    torch.cuda.synchronize()
    bad = [k for k, b in bufs.items() if not b.intact()]
    assert not bad, f"writes outside {bad}"


def test_distillation_and_policy_writes_stay_inside_their_buffers():
    from chunked_lm_head_amd import flce

    dev = gu.device()
    dw_ = synth.distill_custom("guard_distill", T=290, Hs=136, Ht=72, V=1300, chunk_rows=16,
                               ignore_frac=0.1, seed=82)
    x = synth.make_distill_inputs(dw_)
    sh, sw = gu.bf16_tensor(x.s_hidden, dev), gu.bf16_tensor(x.s_weight, dev)
    th, tw = gu.bf16_tensor(x.t_hidden, dev), gu.bf16_tensor(x.t_weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    T, Ds, V = dw_.T, dw_.Hs, dw_.V
    need = flce.distill_workspace_bytes(T, Ds, dw_.Ht, V, dw_.chunk_rows)
    bufs = dict(kl=Guarded((T,), torch.float32, dev), mean=Guarded((), torch.float32, dev),
                dh=Guarded((T, Ds), torch.bfloat16, dev), dw=Guarded((V, Ds), torch.float32, dev),
                ws=Guarded((need,), torch.uint8, dev))
    for div in ("kl", "jsd"):
        flce.distill(sh, sw, th, tw, y, chunk_rows=dw_.chunk_rows,
                     grad_mean=torch.ones((), device=dev), grad_hidden=bufs["dh"].t,
                     grad_weight=bufs["dw"].t, workspace=bufs["ws"].t, kl=bufs["kl"].t,
                     mean=bufs["mean"].t, divergence=div, beta=0.3)
    torch.cuda.synchronize()
    bad = [k for k, b in bufs.items() if not b.intact()]
    assert not bad, f"distillation writes outside {bad}"

    pw = synth.custom("guard_policy", T=384, H=136, V=1100, chunk_rows=32, mode="logprob",
                      reduction="none", seq_len=96, prompt_len=10, seed=83)
    px = synth.make_inputs(pw)
    h, W = gu.bf16_tensor(px.hidden, dev), gu.bf16_tensor(px.weight, dev)
    py = torch.from_numpy(px.labels).to(dev)
    T, D, V, n = pw.T, pw.H, pw.V, 4
    need = flce.policy_workspace_bytes(T, D, V, pw.chunk_rows, n)
    bufs = dict(loss=Guarded((), torch.float32, dev), logp=Guarded((T,), torch.float32, dev),
                dh=Guarded((T, D), torch.bfloat16, dev), dw=Guarded((V, D), torch.float32, dev),
                ws=Guarded((need,), torch.uint8, dev))
    flce.grpo_loss(h, W, py, n, torch.linspace(-1, 1, n, device=dev), beta=0.0,
                   chunk_rows=pw.chunk_rows, grad_loss=torch.ones((), device=dev),
                   grad_hidden=bufs["dh"].t, grad_weight=bufs["dw"].t, workspace=bufs["ws"].t,
                   loss=bufs["loss"].t, logp=bufs["logp"].t)
    torch.cuda.synchronize()
    bad = [k for k, b in bufs.items() if not b.intact()]
    assert not bad, f"policy loss writes outside {bad}"
