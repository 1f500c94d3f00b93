"""GRPO, DPO and KTO on the HIP path vs the CPU oracle.

The loss and the per-token log-probs within 2e-3 absolute; dH and dW within 1e-2
relative Frobenius error, as for the cross-entropy path (the losses reach the LM
head through its log-prob backward).  Side inputs are built from the oracle's
log-probs plus seeded noise: old log-probs give ratios near 1 (some clipped),
reference sequence log-probs give DPO / KTO margins of order 1.  Ratios within
1e-3 of a clipping bound are moved off it, so the GPU's fp32 log-probs and the
oracle's fp64 ones take the same branch of the surrogate.
"""
import math

import numpy as np
import pytest
import torch

from chunked_lm_head_amd import synth
from oracle import flce_oracle as fo
from oracle import policy_oracle as po

import gpu_util as gu

pytestmark = pytest.mark.gpu

IGN = synth.IGNORE_INDEX
GRAD_LOSS = 1.7

# name, kind, (n_seq, seq_len, prompt_len, D, V, chunk_rows), options
CASES = [
    ("grpo_ragged", "grpo", (3, 300, 40, 256, 5000, 64),
     dict(beta=0.3, eps_low=0.2, eps_high=0.2)),
    ("grpo_on_policy", "grpo", (4, 130, 30, 200, 3001, 256),
     dict(beta=0.0, old=False, ref=False)),
    ("grpo_asymmetric", "grpo", (2, 520, 100, 136, 3001, 256),
     dict(beta=0.04, eps_low=0.2, eps_high=0.28)),
    ("grpo_softcap", "grpo", (3, 200, 20, 128, 2000, 64),
     dict(beta=0.3, transform=(0.0, 0.0, 3.0, 0.8))),
    ("grpo_empty_sequence", "grpo", (3, 100, 10, 64, 700, 256),
     dict(beta=0.3, empty=1)),
    ("grpo_many_sequences", "grpo", (2048, 8, 2, 64, 300, 256), dict(beta=0.3)),
    ("grpo_long_sequence", "grpo", (1, 70000, 1000, 64, 300, 256), dict(beta=0.3)),
    # prompts spanning whole 256-token tiles, which the forward and the backward skip
    ("grpo_prompt_tiles", "grpo", (4, 1024, 600, 136, 3001, 256), dict(beta=0.04)),
    # more than 1,024 token tiles: the forward's tile list is numbered in several groups
    ("grpo_many_tiles", "grpo", (2, 140000, 1000, 32, 300, 256), dict(beta=0.3)),
    ("dpo", "dpo", (4, 300, 50, 256, 5000, 64), dict(beta=0.1)),
    ("dpo_many_pairs", "dpo", (1200, 16, 4, 64, 300, 256), dict(beta=0.5)),
    ("dpo_prompt_tiles", "dpo", (2, 1536, 700, 128, 2000, 64), dict(beta=0.1)),
    ("dpo_scaled", "dpo", (2, 260, 60, 200, 3001, 256),
     dict(beta=0.2, transform=(1.3, 0.0, 0.0, 0.7))),
    ("kto", "kto", (5, 260, 60, 200, 3001, 256),
     dict(beta=0.1, kl_ref=0.2, wd=1.0, wu=1.33)),
    ("kto_no_reference_point", "kto", (3, 300, 40, 256, 5000, 64), dict(beta=0.3)),
    ("kto_negative_reference_point", "kto", (1500, 8, 2, 64, 300, 256),
     dict(beta=0.5, kl_ref=-1.0, wd=0.8, wu=1.2)),
]


def _case(name):
    return next(c for c in CASES if c[0] == name)


def _kink_free(lp, old, eps_low, eps_high, mask):
    """Shift float32 old log-probs until no ratio lies within 1e-3 of a clip bound."""
    old = old.copy()
    for _ in range(10):
        r = np.exp(lp - old.astype(np.float64))
        near = ((np.abs(r - (1 + eps_high)) < 1e-3) | (np.abs(r - (1 - eps_low)) < 1e-3)) & mask
        if not near.any():
            return old
        old[near] += np.float32(0.01)
    raise AssertionError("could not move the ratios off the clipping bounds")


def _prepare(case):
    name, kind, (n_seq, S, prompt, D, V, cr), opt = case
    w = synth.policy_custom(name, n_seq, S, prompt, D, V, chunk_rows=cr,
                            seed=sum(map(ord, name)) % 997)
    x = synth.make_policy_inputs(w)
    labels = x.labels.copy()
    if "empty" in opt:
        b = opt["empty"]
        labels[b * S:(b + 1) * S] = IGN
    tr = None if "transform" not in opt else fo.LogitTransform(*opt["transform"])
    lp = po.logp(x.hidden, x.weight, labels, transform=tr)
    mask = labels != IGN
    side = {}
    beta = opt["beta"]
    if kind == "grpo":
        el, eh = opt.get("eps_low", 0.2), opt.get("eps_high", 0.2)
        side["advantages"] = x.advantages
        if opt.get("old", True):
            old = (lp + 0.15 * x.old_noise).astype(np.float32)
            side["old"] = _kink_free(lp, old, el, eh, mask)
        if opt.get("ref", True):
            side["ref"] = (lp + 0.3 * x.ref_noise).astype(np.float32)
    else:
        pi = np.where(mask, lp, 0.0).reshape(n_seq, S).sum(axis=1)
        # margins beta (ref - pi) of order 1 for DPO pairs and KTO sequences
        side["ref_seq"] = (pi + (1.5 / beta) * x.seq_noise).astype(np.float32)
        if kind == "kto":
            side["desirable"] = x.desirable
    return x, labels, tr, side


def _oracle(kind, x, labels, tr, side, opt):
    n_seq = x.workload.n_seq
    lp = po.logp(x.hidden, x.weight, labels, transform=tr)
    if kind == "grpo":
        r = po.grpo_from_logp(lp, labels, n_seq, side["advantages"], old_logp=side.get("old"),
                              ref_logp=side.get("ref"), beta=opt["beta"],
                              eps_low=opt.get("eps_low", 0.2), eps_high=opt.get("eps_high", 0.2))
    elif kind == "dpo":
        r = po.dpo_from_logp(lp, labels, n_seq, side["ref_seq"], beta=opt["beta"])
    else:
        r = po.kto_from_logp(lp, labels, n_seq, side["ref_seq"], side["desirable"],
                             kl_ref=opt.get("kl_ref", 0.0), beta=opt["beta"],
                             desirable_weight=opt.get("wd", 1.0),
                             undesirable_weight=opt.get("wu", 1.0))
    dh, dw = po.grads(x.hidden, x.weight, labels, r.dlogp, grad_loss=GRAD_LOSS, transform=tr)
    return r, dh, dw


def _run(kind, x, labels, tr, side, opt, *, grads=True, accumulate_into=None):
    from chunked_lm_head_amd import flce

    dev = gu.device()
    w = x.workload
    h = gu.bf16_tensor(x.hidden, dev)
    W = gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(labels).to(dev)

    def t(a):
        return None if a is None else torch.from_numpy(np.asarray(a)).to(dev)

    kw = dict(chunk_rows=w.chunk_rows, transform=gu.binding_transform(tr),
              logp=torch.empty(w.T, dtype=torch.float32, device=dev))
    if grads:
        kw["grad_loss"] = torch.tensor(GRAD_LOSS, dtype=torch.float32, device=dev)
    if accumulate_into is not None:
        kw["grad_weight"] = torch.from_numpy(accumulate_into.astype(np.float32)).to(dev)
        kw["accumulate"] = True
    if kind == "grpo":
        out = flce.grpo_loss(h, W, y, w.n_seq, t(side["advantages"]), old_logp=t(side.get("old")),
                             ref_logp=t(side.get("ref")), beta=opt["beta"],
                             eps_low=opt.get("eps_low", 0.2), eps_high=opt.get("eps_high", 0.2),
                             **kw)
    elif kind == "dpo":
        out = flce.dpo_loss(h, W, y, w.n_seq, t(side["ref_seq"]), beta=opt["beta"], **kw)
    else:
        kl = opt.get("kl_ref")
        kl_t = None if kl is None else torch.tensor(kl, dtype=torch.float32, device=dev)
        out = flce.kto_loss(h, W, y, w.n_seq, t(side["ref_seq"]), t(side["desirable"]),
                            kl_ref=kl_t, beta=opt["beta"], desirable_weight=opt.get("wd", 1.0),
                            undesirable_weight=opt.get("wu", 1.0), **kw)
    torch.cuda.synchronize()
    loss, logp, dh, dw = out
    r = dict(loss=float(loss.cpu()), logp=logp.cpu().numpy())
    if grads:
        r["dh"] = dh.float().cpu().numpy()
        r["dw"] = dw.cpu().numpy()
    return r


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_policy_parity(case):
    name, kind, shape, opt = case
    print(f"case {name}: kind {kind} (n_seq, S, prompt, D, V, chunk_rows) = {shape}", flush=True)
    x, labels, tr, side = _prepare(case)
    got = _run(kind, x, labels, tr, side, opt)
    want, dh, dw = _oracle(kind, x, labels, tr, side, opt)
    e = (abs(got["loss"] - want.loss), gu.max_abs(got["logp"], want.logp),
         gu.rel_fro(got["dh"], dh), gu.rel_fro(got["dw"], dw))
    print(f"  loss {got['loss']:.6f} (oracle {want.loss:.6f}) |d loss| {e[0]:.2e} "
          f"|d logp| {e[1]:.2e} dH rel {e[2]:.2e} dW rel {e[3]:.2e}", flush=True)
    assert e[0] <= gu.OUT_TOL and e[1] <= gu.OUT_TOL, e
    assert e[2] <= gu.GRAD_TOL and e[3] <= gu.GRAD_TOL, e
    off = labels == IGN
    assert np.all(got["logp"][off] == 0.0) and np.all(got["dh"][off] == 0.0)


def test_forward_only_and_accumulate():
    case = _case("grpo_ragged")
    _, kind, _, opt = case
    x, labels, tr, side = _prepare(case)
    full = _run(kind, x, labels, tr, side, opt)
    only = _run(kind, x, labels, tr, side, opt, grads=False)
    assert full["loss"] == only["loss"] and np.array_equal(full["logp"], only["logp"])
    base = np.random.default_rng(9).standard_normal((x.workload.V, x.workload.H))
    acc = _run(kind, x, labels, tr, side, opt, accumulate_into=base)
    assert gu.rel_fro(acc["dw"] - base.astype(np.float32), full["dw"]) <= gu.GRAD_TOL


def test_repeat_calls_give_identical_bits():
    case = _case("dpo")
    _, kind, _, opt = case
    x, labels, tr, side = _prepare(case)
    a = _run(kind, x, labels, tr, side, opt)
    b = _run(kind, x, labels, tr, side, opt)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["dh"], b["dh"]) and np.array_equal(a["dw"], b["dw"])


def test_empty_batch():
    from chunked_lm_head_amd import flce

    dev = gu.device()
    h = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    W = torch.ones((300, 64), dtype=torch.bfloat16, device=dev)
    y = torch.empty(0, dtype=torch.int64, device=dev)
    gw = torch.full((300, 64), 7.0, device=dev)
    one = torch.ones((), dtype=torch.float32, device=dev)
    loss, _, _, dw = flce.grpo_loss(h, W, y, 1, torch.zeros(1, device=dev), grad_loss=one,
                                    grad_weight=gw)
    torch.cuda.synchronize()
    assert float(loss.cpu()) == 0.0 and float(dw.abs().max().cpu()) == 0.0
    assert math.isfinite(float(loss.cpu()))


def test_autograd_wrappers():
    from chunked_lm_head_amd import flce

    dev = gu.device()
    for case in (_case("grpo_ragged"), _case("dpo"), _case("kto")):
        _, kind, _, opt = case
        x, labels, tr, side = _prepare(case)
        want, dh, dw = _oracle(kind, x, labels, tr, side, opt)   # upstream GRAD_LOSS
        h = gu.bf16_tensor(x.hidden, dev).requires_grad_()
        W = gu.bf16_tensor(x.weight, dev).requires_grad_()
        y = torch.from_numpy(labels).to(dev)

        def t(a):
            return torch.from_numpy(np.asarray(a)).to(dev)

        kw = dict(chunk_rows=x.workload.chunk_rows, transform=gu.binding_transform(tr))
        if kind == "grpo":
            loss = flce.grpo_loss_fn(h, W, y, x.workload.n_seq, t(side["advantages"]),
                                     old_logp=t(side["old"]), ref_logp=t(side["ref"]),
                                     beta=opt["beta"], **kw)
        elif kind == "dpo":
            loss = flce.dpo_loss_fn(h, W, y, x.workload.n_seq, t(side["ref_seq"]),
                                    beta=opt["beta"], **kw)
        else:
            loss = flce.kto_loss_fn(h, W, y, x.workload.n_seq, t(side["ref_seq"]),
                                    t(side["desirable"]),
                                    kl_ref=torch.tensor(opt["kl_ref"], dtype=torch.float32,
                                                        device=dev),
                                    beta=opt["beta"], desirable_weight=opt["wd"],
                                    undesirable_weight=opt["wu"], **kw)
        (loss * GRAD_LOSS).backward()
        torch.cuda.synchronize()
        assert abs(float(loss.detach().cpu()) - want.loss) <= gu.OUT_TOL
        assert gu.rel_fro(h.grad.float().cpu().numpy(), dh) <= gu.GRAD_TOL
        assert gu.rel_fro(W.grad.float().cpu().numpy(), dw) <= gu.GRAD_TOL
