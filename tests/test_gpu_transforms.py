"""Logit transforms on the HIP path vs the CPU oracle, element by element.

The transform is the chunked call's multiply / divide / softcap / temperature
(Unsloth GRPO page, section "Chunking der abgeflachten Sequenzlaenge"), taken
per raw logit in that order; the oracle applies it in float64 and takes the
chain rule through it.  Tolerances as in the untransformed parity tests.
"""
import numpy as np
import pytest

from chunked_lm_head_amd import synth
from oracle import flce_oracle as o

import gpu_util as gu

pytestmark = pytest.mark.gpu

IGN = synth.IGNORE_INDEX

CASES = [
    # name, (T, D, V, chunk_rows, ignore_frac, mode, reduction, w_std), (mul, div, cap, temp)
    ("temperature", (300, 256, 5000, 64, 0.07, "nll", "mean", None), (0.0, 0.0, 0.0, 0.7)),
    ("multiply", (520, 200, 3001, 256, 0.0, "logprob", "none", None), (2.5, 0.0, 0.0, 1.0)),
    ("divide", (300, 256, 5000, 64, 0.0, "nll", "mean", None), (0.0, 3.0, 0.0, 1.0)),
    ("softcap_tight", (300, 256, 5000, 64, 0.05, "nll", "mean", 0.2), (0.0, 0.0, 1.5, 1.0)),
    ("softcap_saturating", (64, 1024, 3000, 256, 0.0, "nll", "mean", 1.0),
     (0.0, 0.0, 30.0, 1.0)),
    ("combined", (520, 200, 3001, 256, 0.0, "logprob", "none", 0.3), (1.3, 0.8, 4.0, 0.6)),
    ("combined_many_blocks", (8500, 64, 700, 256, 0.03, "nll", "mean", 0.4),
     (0.0, 2.0, 3.0, 1.4)),
    ("combined_wide_d", (130, 1032, 777, 16, 0.1, "logprob", "mean", None), (0.5, 0.0, 2.0, 0.9)),
]


def _inputs(name, shape):
    T, D, V, cr, ign, mode, red, w_std = shape
    kw = dict(seq_len=260, prompt_len=40) if red == "none" else {}
    w = synth.custom(name, T=T, H=D, V=V, chunk_rows=cr, ignore_frac=ign, mode=mode,
                     reduction=red, w_std=w_std, seed=sum(map(ord, name)) % 997, **kw)
    return synth.make_inputs(w)


def _oracle(x, tr):
    w = x.workload
    f = o.forward(x.hidden, x.weight, x.labels, IGN, w.mode, transform=tr)
    if x.grad_out is not None:
        dh, dw = o.backward(x.hidden, x.weight, x.labels, IGN, w.mode, grad_out=x.grad_out,
                            transform=tr)
    else:
        dh, dw = o.backward(x.hidden, x.weight, x.labels, IGN, w.mode, grad_mean=1.0,
                            transform=tr)
    return f, dh, dw


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_transform_parity(case):
    name, shape, vals = case
    x = _inputs(name, shape)
    tr = o.LogitTransform(*vals)
    print(f"case {name}: shape {shape[:3]} transform {vals}", flush=True)
    r = gu.run(x, transform=vals)
    f, dh, dw = _oracle(x, tr)
    e = (gu.max_abs(r["out"], f.out), gu.max_abs(r["lse"], f.lse), abs(r["mean"] - f.mean),
         gu.rel_fro(r["dh"], dh), gu.rel_fro(r["dw"], dw))
    print(f"  |d out| {e[0]:.2e} |d lse| {e[1]:.2e} |d mean| {e[2]:.2e} "
          f"dH rel {e[3]:.2e} dW rel {e[4]:.2e}", flush=True)
    assert e[0] <= gu.OUT_TOL and e[1] <= gu.OUT_TOL and e[2] <= gu.OUT_TOL, e
    assert e[3] <= gu.GRAD_TOL and e[4] <= gu.GRAD_TOL, e
    ign = x.labels == IGN
    assert np.all(r["out"][ign] == 0.0)
    assert np.all(r["dh"][ign] == 0.0)
    if vals[2] != 0.0:
        # a capped logit row lies in [-cap, cap] / temperature: lse - z_label <= 2 cap / temp + log V
        bound = 2.0 * vals[2] / vals[3] + np.log(x.workload.V) + 1e-3
        nll = np.abs(r["out"][~ign])
        assert np.all(nll <= bound), (nll.max(), bound)


def test_equal_scales_give_identical_bits():
    """multiply 2, divide 0.5 and temperature 0.5 are the same scale of the logits."""
    x = _inputs("same_scale", (300, 256, 5000, 64, 0.05, "nll", "mean", None))
    runs = [gu.run(x, transform=v) for v in
            ((2.0, 0.0, 0.0, 1.0), (0.0, 0.5, 0.0, 1.0), (0.0, 0.0, 0.0, 0.5))]
    for r in runs[1:]:
        for k in ("out", "lse", "dh", "dw"):
            assert np.array_equal(r[k], runs[0][k]), k


def test_huge_softcap_is_the_identity():
    x = _inputs("huge_cap", (300, 256, 5000, 64, 0.05, "nll", "mean", None))
    r = gu.run(x, transform=(0.0, 0.0, 1.0e4, 1.0))
    f, dh, dw = _oracle(x, None)
    assert gu.max_abs(r["out"], f.out) <= gu.OUT_TOL
    assert gu.rel_fro(r["dh"], dh) <= gu.GRAD_TOL
    assert gu.rel_fro(r["dw"], dw) <= gu.GRAD_TOL


def test_autograd_wrapper_passes_the_transform():
    import torch

    from chunked_lm_head_amd import flce

    x = _inputs("autograd_xf", (260, 128, 2000, 256, 0.0, "logprob", "none", 0.3))
    dev = gu.device()
    h = gu.bf16_tensor(x.hidden, dev).requires_grad_()
    W = gu.bf16_tensor(x.weight, dev).requires_grad_()
    y = torch.from_numpy(x.labels).to(dev)
    kw = dict(logit_softcapping=2.0, temperature=0.8)
    lp = flce.selective_log_softmax(h, W, y, **kw)
    g = torch.from_numpy(x.grad_out).to(dev)
    (lp * g).sum().backward()
    torch.cuda.synchronize()
    tr = o.LogitTransform(softcap=2.0, temperature=0.8)
    f = o.forward(x.hidden, x.weight, x.labels, IGN, "logprob", transform=tr)
    dh, dw = o.backward(x.hidden, x.weight, x.labels, IGN, "logprob", grad_out=x.grad_out,
                        transform=tr)
    assert gu.max_abs(lp.detach().cpu().numpy(), f.out) <= gu.OUT_TOL
    assert gu.rel_fro(h.grad.float().cpu().numpy(), dh) <= gu.GRAD_TOL
    # the wrapper returns dW in the weight's dtype (bf16)
    assert gu.rel_fro(W.grad.float().cpu().numpy(), dw) <= gu.GRAD_TOL
