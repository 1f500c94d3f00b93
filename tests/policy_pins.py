"""Pins for the policy-loss oracle (GRPO, DPO, KTO on the selective log-softmax).

Each ``check_*`` takes the policy oracle module and raises AssertionError when
it disagrees with an independent fact:

* closed forms worked by hand: on-policy GRPO is minus the mean advantage; the
  four clipping cases of the GRPO surrogate (ratio 2 and 1/2, advantage of
  either sign); the KL estimator at ref - logp = ln 2 is 1 - ln 2; DPO at equal
  margins is ln 2 per pair; KTO at r = z0 is half the weight;
* the KL estimator is non-negative, DPO is symmetric under swapping chosen and
  rejected with the sign of the margin, KTO clamps a negative reference point;
* central finite differences of each loss in the per-token log-probs check
  dL/dlogp, and through the LM head (the cross-entropy oracle, pinned on its
  own) check dH and dW;
* brute force: a tiny DPO case computed with Python's ``math`` over exactly
  decoded bf16 values, no numpy.
"""
from __future__ import annotations

import math

import numpy as np

from chunked_lm_head_amd import synth

from oracle_pins import py_decode

IGN = -100


def _labels(n_seq, S, V, masked, seed=0):
    rng = np.random.default_rng(seed)
    y = rng.integers(0, V, size=n_seq * S).astype(np.int64)
    for t in masked:
        y[t] = IGN
    return y


def check_grpo_on_policy_is_minus_mean_advantage(p):
    n_seq, S = 4, 5
    y = _labels(n_seq, S, 50, masked=[0, 1, 7] + list(range(15, 20)))  # sequence 3 empty
    lp = -np.linspace(0.5, 3.0, n_seq * S)
    A = np.array([0.5, -1.25, 2.0, 9.0])
    r = p.grpo_from_logp(lp, y, n_seq, A)
    used = [0, 1, 2]
    assert abs(r.loss - (-(0.5 - 1.25 + 2.0) / 3)) < 1e-15, r.loss
    n = [3, 4, 5]
    for b in used:
        for t in range(b * S, (b + 1) * S):
            want = 0.0 if y[t] == IGN else -A[b] / (3 * n[b])
            assert abs(r.dlogp[t] - want) < 1e-15, (t, r.dlogp[t], want)
    assert np.all(r.dlogp[15:] == 0.0)


def _one(p, ratio, A, eps_low=0.2, eps_high=0.2, **kw):
    y = np.array([3], dtype=np.int64)
    lp = np.array([-1.7])
    old = lp - math.log(ratio)
    return p.grpo_from_logp(lp, y, 1, np.array([A]), old_logp=old, eps_low=eps_low,
                            eps_high=eps_high, **kw)


def check_grpo_clipping_cases(p):
    # ratio 2 above 1 + eps: a positive advantage is clipped (no gradient), a negative one is not
    r = _one(p, 2.0, 1.0)
    assert abs(r.loss + 1.2) < 1e-12 and r.dlogp[0] == 0.0, (r.loss, r.dlogp)
    r = _one(p, 2.0, -1.0)
    assert abs(r.loss - 2.0) < 1e-12 and abs(r.dlogp[0] - 2.0) < 1e-12, (r.loss, r.dlogp)
    # ratio 1/2 below 1 - eps: the opposite
    r = _one(p, 0.5, 1.0)
    assert abs(r.loss + 0.5) < 1e-12 and abs(r.dlogp[0] + 0.5) < 1e-12, (r.loss, r.dlogp)
    r = _one(p, 0.5, -1.0)
    assert abs(r.loss - 0.8) < 1e-12 and r.dlogp[0] == 0.0, (r.loss, r.dlogp)
    # asymmetric range [0.9, 1.3]: 1.25 is inside, 0.85 is below
    r = _one(p, 1.25, 1.0, eps_low=0.1, eps_high=0.3)
    assert abs(r.loss + 1.25) < 1e-12 and abs(r.dlogp[0] + 1.25) < 1e-12
    r = _one(p, 0.85, -2.0, eps_low=0.1, eps_high=0.3)
    assert abs(r.loss - 1.8) < 1e-12 and r.dlogp[0] == 0.0, (r.loss, r.dlogp)


def check_grpo_kl_term(p):
    y = np.array([3, 4], dtype=np.int64)
    lp = np.array([-1.0, -2.5])
    A = np.array([0.0])
    r = p.grpo_from_logp(lp, y, 1, A, ref_logp=lp, beta=0.7)
    assert r.loss == 0.0 and np.all(r.dlogp == 0.0)
    ref = lp + math.log(2.0)
    r = p.grpo_from_logp(lp, y, 1, A, ref_logp=ref, beta=0.5)
    # k = 2 - ln 2 - 1 per token, J = -beta k, L = beta (1 - ln 2); dk/dlogp = 1 - 2 = -1
    assert abs(r.loss - 0.5 * (1.0 - math.log(2.0))) < 1e-15, r.loss
    assert np.allclose(r.dlogp, -0.5 * 1.0 / 2.0, rtol=0, atol=1e-15), r.dlogp
    rng = np.random.default_rng(4)
    lp = -rng.uniform(0.1, 5.0, 200)
    ref = lp + rng.normal(0.0, 2.0, 200)
    y = np.zeros(200, dtype=np.int64)
    for t in range(200):  # every single-token KL estimate is >= 0
        r = p.grpo_from_logp(lp[t:t + 1], y[:1], 1, A, ref_logp=ref[t:t + 1], beta=1.0)
        assert r.loss >= 0.0, (t, r.loss)


def check_dpo_closed_forms(p):
    n_seq, S = 4, 3
    y = _labels(n_seq, S, 20, masked=[0, 6])
    lp = -np.array([1.0, 2.0, 0.5, 1.5, 0.25, 3.0, 2.0, 1.0, 0.75, 0.5, 0.5, 0.5])
    pi = [np.where(y[b * S:(b + 1) * S] != IGN, lp[b * S:(b + 1) * S], 0.0).sum()
          for b in range(n_seq)]
    beta = 0.3
    # pair 0: equal margins; pair 1: the chosen margin 4 above the rejected one
    ref = np.array([pi[0] - 1.0, pi[1] - 4.0, pi[2] - 1.0, pi[3]])
    r = p.dpo_from_logp(lp, y, n_seq, ref, beta=beta)
    d1 = beta * 4.0
    want = (math.log(2.0) + math.log1p(math.exp(-d1))) / 2
    assert abs(r.loss - want) < 1e-14, (r.loss, want)
    g0, g1 = beta * 0.5 / 2, beta / (1.0 + math.exp(d1)) / 2
    for b, g in ((0, -g0), (1, -g1), (2, g0), (3, g1)):
        for t in range(b * S, (b + 1) * S):
            want = 0.0 if y[t] == IGN else g
            assert abs(r.dlogp[t] - want) < 1e-15, (b, t, r.dlogp[t], want)
    # swapping chosen and rejected flips the margins
    sw = np.r_[S * 2:S * 4, 0:S * 2]
    r2 = p.dpo_from_logp(lp[sw], y[sw], n_seq, np.r_[ref[2:], ref[:2]], beta=beta)
    want = (math.log(2.0) + math.log1p(math.exp(d1))) / 2
    assert abs(r2.loss - want) < 1e-14, (r2.loss, want)


def check_kto_closed_forms(p):
    n_seq, S = 3, 4
    y = _labels(n_seq, S, 20, masked=[1, 2, 11])
    lp = -np.arange(1, 13) / 4.0
    pi = np.array([np.where(y[b * S:(b + 1) * S] != IGN, lp[b * S:(b + 1) * S], 0.0).sum()
                   for b in range(n_seq)])
    des = np.array([1, 0, 1])
    beta, ld, lu, z0 = 0.2, 1.5, 0.75, 0.4
    r = p.kto_from_logp(lp, y, n_seq, pi - z0, des, kl_ref=z0, beta=beta,
                        desirable_weight=ld, undesirable_weight=lu)
    lam = np.array([ld, lu, ld])
    assert abs(r.loss - lam.sum() / 2 / 3) < 1e-15, r.loss
    # sigmoid'(0) = 1/4: desirable -lam beta / 4 / B, undesirable +lam beta / 4 / B
    for b in range(n_seq):
        g = (-1 if des[b] else 1) * lam[b] * beta / 4 / 3
        for t in range(b * S, (b + 1) * S):
            want = 0.0 if y[t] == IGN else g
            assert abs(r.dlogp[t] - want) < 1e-15, (b, t, r.dlogp[t], want)
    # a negative reference point counts as 0
    a = p.kto_from_logp(lp, y, n_seq, pi - 0.3, des, kl_ref=-2.0, beta=beta)
    b = p.kto_from_logp(lp, y, n_seq, pi - 0.3, des, kl_ref=0.0, beta=beta)
    assert a.loss == b.loss and np.array_equal(a.dlogp, b.dlogp)
    # one desirable sequence with margin m: 1 - sigmoid(beta m), by hand
    r = p.kto_from_logp(lp[:S], y[:S], 1, np.array([pi[0] - 3.0]), np.array([1]), beta=0.5)
    assert abs(r.loss - (1.0 - 1.0 / (1.0 + math.exp(-1.5)))) < 1e-15, r.loss


def _fd(f, x, i, eps=1e-6):
    old = x[i]
    x[i] = old + eps
    a = f(x)
    x[i] = old - eps
    b = f(x)
    x[i] = old
    return (a - b) / (2 * eps)


def check_finite_differences_in_logp(p):
    rng = np.random.default_rng(11)
    n_seq, S = 4, 6
    y = _labels(n_seq, S, 30, masked=[0, 5, 13, 14])
    lp = -rng.uniform(0.2, 4.0, n_seq * S)
    old = lp + rng.normal(0.0, 0.15, n_seq * S)
    ref = lp + rng.normal(0.0, 0.3, n_seq * S)
    A = rng.normal(0.0, 1.0, n_seq)
    kinks = np.abs(np.abs(np.exp(lp - old) - 1.0) - 0.2) < 1e-3
    assert not kinks.any()
    rng_ref = rng.normal(-10.0, 2.0, n_seq)
    cases = [
        lambda x: p.grpo_from_logp(x, y, n_seq, A, old_logp=old, ref_logp=ref, beta=0.3),
        lambda x: p.dpo_from_logp(x, y, n_seq, rng_ref, beta=0.4),
        lambda x: p.kto_from_logp(x, y, n_seq, rng_ref, [1, 0, 0, 1], kl_ref=0.3, beta=0.7,
                                  desirable_weight=1.2, undesirable_weight=0.6),
    ]
    for case in cases:
        d = case(lp.copy()).dlogp
        for i in range(n_seq * S):
            num = _fd(lambda x: case(x).loss, lp.copy(), i)
            assert abs(num - d[i]) < 1e-8 + 1e-6 * abs(num), (i, num, d[i])


def _tiny_head(seed, T, D, V, w_std=0.6):
    w = synth.custom("pin", T=T, H=D, V=V, w_std=w_std, seed=seed)
    x = synth.make_inputs(w)
    from oracle import flce_oracle as fo
    return fo.decode_bf16(x.hidden), fo.decode_bf16(x.weight), x.labels.copy()


def check_finite_differences_through_the_head(p):
    from oracle import flce_oracle as fo
    n_seq, S, D, V = 2, 4, 5, 7
    h, w, y = _tiny_head(21, n_seq * S, D, V)
    y[[0, 5]] = IGN
    rng = np.random.default_rng(5)
    base = p.logp(h, w, y)
    old = base + rng.normal(0.0, 0.1, n_seq * S)
    ref = base + rng.normal(0.0, 0.2, n_seq * S)
    A = np.array([0.8, -1.1])
    tr = fo.LogitTransform(softcap=2.5, temperature=0.8)
    losses = [
        lambda lp: p.grpo_from_logp(lp, y, n_seq, A, old_logp=old, ref_logp=ref, beta=0.2),
        lambda lp: p.dpo_from_logp(lp, y, n_seq, np.array([-9.0, -11.0]), beta=0.5),
        lambda lp: p.kto_from_logp(lp, y, n_seq, np.array([-9.0, -11.0]), [0, 1], kl_ref=0.1,
                                   beta=0.5),
    ]
    for transform in (None, tr):
        for L in losses:
            dlogp = L(p.logp(h, w, y, transform=transform)).dlogp
            dh, dw = p.grads(h, w, y, dlogp, grad_loss=1.7, transform=transform)

            def total(hh, ww):
                return 1.7 * L(p.logp(hh, ww, y, transform=transform)).loss

            for arr, grad in ((h, dh), (w, dw)):
                for i in [(0, 1), (3, 4), (6, 0), (2, 2)]:
                    if i[0] >= arr.shape[0]:
                        continue
                    old_v = arr[i]
                    arr[i] = old_v + 1e-6
                    a = total(h, w)
                    arr[i] = old_v - 1e-6
                    b = total(h, w)
                    arr[i] = old_v
                    num = (a - b) / 2e-6
                    assert abs(num - grad[i]) < 1e-8 + 1e-5 * abs(num), (i, num, grad[i])
    # ignored tokens get no dH row
    dh, _ = p.grads(h, w, y, losses[0](p.logp(h, w, y)).dlogp)
    assert np.all(dh[[0, 5]] == 0.0)


def check_dpo_brute_force(p):
    n_seq, S, D, V = 2, 3, 4, 6
    w = synth.custom("pin", T=n_seq * S, H=D, V=V, w_std=0.7, seed=31)
    x = synth.make_inputs(w)
    y = x.labels.copy()
    y[1] = IGN
    hs = [py_decode(x.hidden[t]) for t in range(n_seq * S)]
    ws = [py_decode(x.weight[v]) for v in range(V)]
    lp = []
    for t in range(n_seq * S):
        z = [math.fsum(a * b for a, b in zip(hs[t], ws[v])) for v in range(V)]
        lse = math.log(math.fsum(math.exp(zv) for zv in z))
        lp.append(0.0 if y[t] == IGN else z[y[t]] - lse)
    pi = [math.fsum(lp[b * S:(b + 1) * S]) for b in range(n_seq)]
    ref = [-5.0, -6.5]
    beta = 0.8
    d = beta * ((pi[0] - ref[0]) - (pi[1] - ref[1]))
    want = math.log1p(math.exp(-d))
    got = p.dpo_from_logp(p.logp(x.hidden, x.weight, y), y, n_seq, np.array(ref), beta=beta)
    assert abs(got.loss - want) < 1e-12, (got.loss, want)


ALL_CHECKS = [
    check_grpo_on_policy_is_minus_mean_advantage,
    check_grpo_clipping_cases,
    check_grpo_kl_term,
    check_dpo_closed_forms,
    check_kto_closed_forms,
    check_finite_differences_in_logp,
    check_finite_differences_through_the_head,
    check_dpo_brute_force,
]
