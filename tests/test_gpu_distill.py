"""Distillation (KL and the generalized JSD) on the HIP path vs the CPU oracle, element by element.

Per-token KL and the mean within 2e-3 absolute; the student's dH and dW within
1e-2 relative Frobenius error (G is rounded to bf16 before the backward GEMMs,
dH is returned in bf16), as for the cross-entropy path.
"""
import numpy as np
import pytest
import torch

from chunked_lm_head_amd import synth
from oracle import distill_oracle as d
from oracle import flce_oracle as fo

import gpu_util as gu

pytestmark = pytest.mark.gpu

IGN = synth.IGNORE_INDEX

CASES = [
    # name, (T, Ds, Dt, V, chunk_rows, ignore_frac, reduction, ws, wt), transform, mask
    ("tiny", None, None, True),
    ("ragged", (300, 256, 384, 5000, 64, 0.07, "mean", None, None), None, True),
    ("per_token_grad", (520, 200, 136, 3001, 256, 0.0, "none", 0.3, 0.3), None, True),
    ("many_blocks", (8500, 64, 128, 700, 256, 0.03, "mean", 0.4, 0.4), None, True),
    ("wide", (130, 1032, 520, 777, 16, 0.1, "none", None, None), None, True),
    ("no_mask", (300, 256, 384, 5000, 64, 0.0, "mean", None, None), None, False),
    ("softcap_temperature", (300, 256, 384, 5000, 64, 0.05, "mean", 0.2, 0.2),
     (0.0, 0.0, 1.5, 0.7), True),
    ("scaled", (520, 200, 136, 3001, 256, 0.0, "none", 0.3, 0.3), (1.3, 0.8, 0.0, 0.6), True),
    # the largest hidden size accepted, on the student (the block shape follows max(Ds, Dt))
    ("max_d", (200, 65536, 1024, 600, 64, 0.05, "mean", None, None), None, True),
]


def _inputs(name, shape):
    if shape is None:
        return synth.make_distill_inputs(synth.DISTILL_WORKLOADS["distill_" + name])
    T, Ds, Dt, V, cr, ign, red, ws, wt = shape
    w = synth.distill_custom(name, T=T, Hs=Ds, Ht=Dt, V=V, chunk_rows=cr, ws_std=ws, wt_std=wt,
                             ignore_frac=ign, reduction=red, seed=sum(map(ord, name)) % 991)
    return synth.make_distill_inputs(w)


def _tensors(x, dev):
    return (gu.bf16_tensor(x.s_hidden, dev), gu.bf16_tensor(x.s_weight, dev),
            gu.bf16_tensor(x.t_hidden, dev), gu.bf16_tensor(x.t_weight, dev))


def _run(x, *, mask=True, transform=None, grads=True, accumulate_into=None, divergence="kl",
         beta=0.5):
    from chunked_lm_head_amd import flce

    dev = gu.device()
    sh, sw, th, tw = _tensors(x, dev)
    labels = torch.from_numpy(x.labels).to(dev) if mask else None
    kw = {}
    if grads:
        if x.grad_out is not None:
            kw["grad_out"] = torch.from_numpy(x.grad_out).to(dev)
        else:
            kw["grad_mean"] = torch.ones((), dtype=torch.float32, device=dev)
    gw = None
    if accumulate_into is not None:
        gw = torch.from_numpy(accumulate_into.astype(np.float32)).to(dev)
        kw["grad_weight"] = gw
        kw["accumulate"] = True
    kl, mean, dh, dw = flce.distill(sh, sw, th, tw, labels,
                                    chunk_rows=x.workload.chunk_rows,
                                    transform=gu.binding_transform(transform),
                                    divergence=divergence, beta=beta, **kw)
    torch.cuda.synchronize()
    r = dict(kl=kl.cpu().numpy(), mean=float(mean.cpu()))
    if grads:
        r["dh"] = dh.float().cpu().numpy()
        r["dw"] = dw.cpu().numpy()
    return r


def _oracle(x, *, mask=True, transform=None, divergence="kl", beta=0.5):
    tr = None if transform is None else fo.LogitTransform(*transform)
    labels = x.labels if mask else None
    kw = dict(transform=tr, divergence=divergence, beta=beta)
    f = d.forward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, labels, **kw)
    if x.grad_out is not None:
        dh, dw = d.backward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, labels,
                            grad_out=x.grad_out, **kw)
    else:
        dh, dw = d.backward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, labels,
                            grad_mean=1.0, **kw)
    return f, dh, dw


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_distill_parity(case):
    name, shape, transform, mask = case
    x = _inputs(name, shape)
    w = x.workload
    print(f"case {name}: T={w.T} Ds={w.Hs} Dt={w.Ht} V={w.V} transform {transform}", flush=True)
    r = _run(x, mask=mask, transform=transform)
    f, dh, dw = _oracle(x, mask=mask, transform=transform)
    e = (gu.max_abs(r["kl"], f.kl), abs(r["mean"] - f.mean), gu.rel_fro(r["dh"], dh),
         gu.rel_fro(r["dw"], dw))
    print(f"  |d kl| {e[0]:.2e} |d mean| {e[1]:.2e} dH rel {e[2]:.2e} dW rel {e[3]:.2e}",
          flush=True)
    assert e[0] <= gu.OUT_TOL and e[1] <= gu.OUT_TOL, e
    assert e[2] <= gu.GRAD_TOL and e[3] <= gu.GRAD_TOL, e
    if mask:
        m = x.labels == IGN
        assert np.all(r["kl"][m] == 0.0)
        assert np.all(r["dh"][m] == 0.0)


JSD_CASES = [
    # (case of CASES, beta)
    ("tiny", 0.5), ("ragged", 0.5), ("per_token_grad", 0.1), ("many_blocks", 0.9),
    ("wide", 0.5), ("no_mask", 0.3), ("softcap_temperature", 0.5), ("scaled", 0.7),
]


@pytest.mark.parametrize("name,beta", JSD_CASES, ids=lambda v: str(v))
def test_jsd_parity(name, beta):
    case = [c for c in CASES if c[0] == name][0]
    _, shape, transform, mask = case
    x = _inputs(name, shape)
    w = x.workload
    print(f"case jsd {name} beta {beta}: T={w.T} Ds={w.Hs} Dt={w.Ht} V={w.V} transform "
          f"{transform}", flush=True)
    r = _run(x, mask=mask, transform=transform, divergence="jsd", beta=beta)
    f, dh, dw = _oracle(x, mask=mask, transform=transform, divergence="jsd", beta=beta)
    e = (gu.max_abs(r["kl"], f.kl), abs(r["mean"] - f.mean), gu.rel_fro(r["dh"], dh),
         gu.rel_fro(r["dw"], dw))
    print(f"  |d jsd| {e[0]:.2e} |d mean| {e[1]:.2e} dH rel {e[2]:.2e} dW rel {e[3]:.2e}",
          flush=True)
    assert e[0] <= gu.OUT_TOL and e[1] <= gu.OUT_TOL, e
    assert e[2] <= gu.GRAD_TOL and e[3] <= gu.GRAD_TOL, e
    if mask:
        m = x.labels == IGN
        assert np.all(r["kl"][m] == 0.0) and np.all(r["dh"][m] == 0.0)


def test_jsd_forward_only_matches_and_identical_heads_vanish():
    x = _inputs("jfo", (300, 256, 384, 5000, 64, 0.05, "mean", None, None))
    full = _run(x, divergence="jsd", beta=0.4)
    only = _run(x, grads=False, divergence="jsd", beta=0.4)
    assert np.array_equal(full["kl"], only["kl"]) and full["mean"] == only["mean"]
    y = _inputs("jsame", (300, 256, 256, 5000, 64, 0.05, "mean", None, None))
    y.t_hidden, y.t_weight = y.s_hidden, y.s_weight
    r = _run(y, divergence="jsd", beta=0.5)
    # p_t = p_s bit for bit; beta p + (1 - beta) p rounds to p within an ulp
    assert np.abs(r["kl"]).max() <= 1e-6, np.abs(r["kl"]).max()
    assert np.abs(r["dw"]).max() <= 1e-6, np.abs(r["dw"]).max()


def test_identical_heads_give_exact_zero():
    x = _inputs("same", (300, 256, 256, 5000, 64, 0.05, "mean", None, None))
    x.t_hidden, x.t_weight = x.s_hidden, x.s_weight
    r = _run(x)
    assert np.all(r["kl"] == 0.0), np.abs(r["kl"]).max()
    assert np.all(r["dh"] == 0.0) and np.all(r["dw"] == 0.0)


def test_forward_only_matches_and_accumulate():
    x = _inputs("fo", (300, 256, 384, 5000, 64, 0.05, "mean", None, None))
    full = _run(x)
    only = _run(x, grads=False)
    assert np.array_equal(full["kl"], only["kl"]) and full["mean"] == only["mean"]
    base = np.random.default_rng(3).standard_normal((5000, 256)).astype(np.float32)
    acc = _run(x, accumulate_into=base)
    # fp32 rounding of base (~1) + dW (~1e-5) leaves ~1e-3 relative error on the added part
    assert gu.rel_fro(acc["dw"] - base, full["dw"]) <= gu.GRAD_TOL


def test_autograd_wrapper():
    from chunked_lm_head_amd import flce

    x = _inputs("ag", (260, 128, 192, 2000, 64, 0.1, "none", 0.3, 0.3))
    dev = gu.device()
    sh, sw, th, tw = _tensors(x, dev)
    labels = torch.from_numpy(x.labels).to(dev)
    g = torch.from_numpy(x.grad_out).to(dev)
    f, dh, dw = _oracle(x, transform=(0.0, 0.0, 0.0, 0.8))
    for reduction in ("none", "mean"):
        a = sh.clone().requires_grad_()
        b = sw.clone().requires_grad_()
        out = flce.chunked_distill_kl(a, b, th, tw, labels, chunk_rows=64, reduction=reduction,
                                      temperature=0.8)
        if reduction == "none":
            (out * g).sum().backward()
            odh, odw = dh, dw
            assert gu.max_abs(out.detach().cpu().numpy(), f.kl) <= gu.OUT_TOL
        else:
            (out * 2.5).backward()
            odh, odw = d.backward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, x.labels,
                                  grad_mean=2.5, transform=fo.LogitTransform(temperature=0.8))
            assert abs(float(out.detach().cpu()) - f.mean) <= gu.OUT_TOL
        torch.cuda.synchronize()
        assert gu.rel_fro(a.grad.float().cpu().numpy(), odh) <= gu.GRAD_TOL
        assert gu.rel_fro(b.grad.float().cpu().numpy(), odw) <= gu.GRAD_TOL


def test_autograd_wrapper_jsd():
    from chunked_lm_head_amd import flce

    x = _inputs("agj", (260, 128, 192, 2000, 64, 0.1, "none", 0.3, 0.3))
    dev = gu.device()
    sh, sw, th, tw = _tensors(x, dev)
    labels = torch.from_numpy(x.labels).to(dev)
    f, _, _ = _oracle(x, divergence="jsd", beta=0.3)
    odh, odw = d.backward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, x.labels,
                          grad_mean=2.5, divergence="jsd", beta=0.3)
    a = sh.clone().requires_grad_()
    b = sw.clone().requires_grad_()
    out = flce.chunked_distill_kl(a, b, th, tw, labels, chunk_rows=64, divergence="jsd",
                                  beta=0.3)
    (out * 2.5).backward()
    torch.cuda.synchronize()
    assert abs(float(out.detach().cpu()) - f.mean) <= gu.OUT_TOL
    assert gu.rel_fro(a.grad.float().cpu().numpy(), odh) <= gu.GRAD_TOL
    assert gu.rel_fro(b.grad.float().cpu().numpy(), odw) <= gu.GRAD_TOL


def test_empty_batch():
    from chunked_lm_head_amd import flce

    dev = gu.device()
    sh = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    th = torch.empty((0, 128), dtype=torch.bfloat16, device=dev)
    sw = torch.ones((300, 64), dtype=torch.bfloat16, device=dev)
    tw = torch.ones((300, 128), dtype=torch.bfloat16, device=dev)
    gw = torch.full((300, 64), 7.0, device=dev)
    kl, mean, dh, dw = flce.distill(sh, sw, th, tw, grad_mean=torch.ones((), device=dev),
                                    grad_weight=gw)
    torch.cuda.synchronize()
    assert float(mean.cpu()) == 0.0
    assert float(gw.abs().max().cpu()) == 0.0
