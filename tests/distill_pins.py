"""Pins for the distillation oracle: facts fixed by mathematics and by the
already-pinned cross-entropy oracle.

Each ``check_*`` takes the distillation oracle module and raises
AssertionError when it disagrees with an independent fact:

* identical student and teacher heads: KL = 0 and zero gradients;
* a zero teacher lm_head makes the teacher uniform: KL = lse_s - mean_v zs - ln V,
  brute-forced with Python's ``math.fsum`` over exactly decoded bf16 values;
* a teacher that puts all its mass on one label: KL -> the student's NLL of
  that label and the gradients -> the cross-entropy gradients (the
  cross-entropy oracle is pinned on its own);
* two classes: the Bernoulli KL written with ``math.log``;
* central finite differences of the mean KL check dHs and dWs, with and
  without a logit transform;
* masked tokens contribute nothing; the per-row helpers agree with the full
  forward and backward; without a transform the gradient rows sum to zero;
* the generalized JSD: zero for identical heads, symmetric and within [0, ln 2]
  at beta = 1/2 (ln 2 for disjoint supports), JSD_beta / beta and
  JSD_beta / (1 - beta) tend to the forward and reverse KL, the two-class case
  written with ``math``, finite differences, and the row helpers.
"""
from __future__ import annotations

import math

import numpy as np

from chunked_lm_head_amd import synth
from oracle import flce_oracle as fo

from oracle_pins import bf16_exact, py_decode, small_blocks

IGN = -100


def _case(T, Hs, Ht, V, seed, ws=0.5, wt=0.5, ignore_frac=0.0, reduction="mean"):
    w = synth.distill_custom("pin", T=T, Hs=Hs, Ht=Ht, V=V, ws_std=ws, wt_std=wt,
                             ignore_frac=ignore_frac, reduction=reduction, seed=seed)
    return synth.make_distill_inputs(w)


def check_identical_heads(d):
    x = _case(9, 16, 16, 37, seed=3)
    f = d.forward(x.s_hidden, x.s_weight, x.s_hidden, x.s_weight)
    assert np.max(np.abs(f.kl)) < 1e-12, f.kl
    assert np.allclose(f.lse_s, f.lse_t, rtol=0, atol=0)
    dh, dw = d.backward(x.s_hidden, x.s_weight, x.s_hidden, x.s_weight)
    assert np.max(np.abs(dh)) < 1e-14 and np.max(np.abs(dw)) < 1e-14


def check_uniform_teacher(d):
    T, Hs, Ht, V = 4, 6, 5, 11
    x = _case(T, Hs, Ht, V, seed=5, ws=0.75)
    tw = np.zeros((V, Ht), dtype=np.uint16)
    f = d.forward(x.s_hidden, x.s_weight, x.t_hidden, tw)
    hs = [py_decode(x.s_hidden[t]) for t in range(T)]
    ws = [py_decode(x.s_weight[v]) for v in range(V)]
    for t in range(T):
        z = [math.fsum(a * b for a, b in zip(hs[t], ws[v])) for v in range(V)]
        lse = math.log(math.fsum(math.exp(zv) for zv in z))
        want = lse - math.fsum(z) / V - math.log(V)
        assert abs(f.kl[t] - want) < 1e-12, (t, f.kl[t], want)


def _onehot_teacher(T, Ht, V, labels, big=64.0):
    """Teacher hidden = e_0 and lm_head column 0 = big at each token's label.

    Needs distinct labels per token so that one lm_head column can serve all
    (each token's hidden selects its own column)."""
    th = np.zeros((T, Ht), dtype=np.uint16)
    tw = np.zeros((V, Ht), dtype=np.uint16)
    one = bf16_exact([1.0])[0]
    b = bf16_exact([big])[0]
    for t in range(T):
        th[t, t] = one
        tw[labels[t], t] = b
    return th, tw


def check_onehot_teacher_is_cross_entropy(d):
    T, Hs, V = 5, 12, 40
    Ht = T
    x = _case(T, Hs, Ht, V, seed=7)
    labels = np.array([3, 17, 0, 39, 22], dtype=np.int64)
    th, tw = _onehot_teacher(T, Ht, V, labels)
    f = d.forward(x.s_hidden, x.s_weight, th, tw)
    ce = fo.forward(x.s_hidden, x.s_weight, labels)
    # pt(label) = 1 - (V - 1) e^-64: KL = NLL up to ~1e-26
    assert np.allclose(f.kl, ce.out, rtol=1e-12, atol=1e-12), (f.kl, ce.out)
    dh, dw = d.backward(x.s_hidden, x.s_weight, th, tw)
    ch, cw = fo.backward(x.s_hidden, x.s_weight, labels)
    assert np.allclose(dh, ch, rtol=1e-10, atol=1e-14)
    assert np.allclose(dw, cw, rtol=1e-10, atol=1e-14)


def check_two_class(d):
    T, Hs, Ht, V = 6, 8, 7, 2
    x = _case(T, Hs, Ht, V, seed=11, ws=1.0, wt=1.0)
    f = d.forward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight)
    hs = [py_decode(x.s_hidden[t]) for t in range(T)]
    ht = [py_decode(x.t_hidden[t]) for t in range(T)]
    ws = [py_decode(x.s_weight[v]) for v in range(V)]
    wt = [py_decode(x.t_weight[v]) for v in range(V)]
    for t in range(T):
        ds = math.fsum(a * b for a, b in zip(hs[t], ws[1])) - math.fsum(
            a * b for a, b in zip(hs[t], ws[0]))
        dt = math.fsum(a * b for a, b in zip(ht[t], wt[1])) - math.fsum(
            a * b for a, b in zip(ht[t], wt[0]))
        q = 1.0 / (1.0 + math.exp(-ds))   # student p(class 1)
        p = 1.0 / (1.0 + math.exp(-dt))   # teacher p(class 1)
        want = p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q))
        assert abs(f.kl[t] - want) < 1e-12, (t, f.kl[t], want)
        assert f.kl[t] >= 0.0


def _fd_check(d, transform):
    x = _case(5, 6, 7, 13, seed=13, ws=0.8, wt=0.8)
    hs = fo.decode_bf16(x.s_hidden)
    ws = fo.decode_bf16(x.s_weight)
    ht = fo.decode_bf16(x.t_hidden)
    wt = fo.decode_bf16(x.t_weight)
    labels = np.array([0, IGN, 0, 0, 0], dtype=np.int64)

    def loss(h, w):
        return d.forward(h, w, ht, wt, labels, transform=transform).mean

    dh, dw = d.backward(hs, ws, ht, wt, labels, transform=transform)
    eps = 1e-6
    rng = np.random.default_rng(0)
    for arr, grad in ((hs, dh), (ws, dw)):
        for _ in range(12):
            i = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[i]
            arr[i] = old + eps
            lp = loss(hs, ws)
            arr[i] = old - eps
            lm = loss(hs, ws)
            arr[i] = old
            num = (lp - lm) / (2 * eps)
            assert abs(num - grad[i]) < 1e-7 + 1e-6 * abs(num), (i, num, grad[i])
    assert np.all(dh[1] == 0.0)


def check_finite_differences(d):
    _fd_check(d, None)


def check_finite_differences_transformed(d):
    _fd_check(d, fo.LogitTransform(scale_multiply=1.3, softcap=1.5, temperature=0.7))


def check_mask_and_mean(d):
    x = _case(11, 8, 9, 30, seed=17, ignore_frac=0.3)
    f = d.forward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, x.labels)
    m = x.labels == IGN
    assert m.sum() == 3
    assert np.all(f.kl[m] == 0.0) and np.all(f.kl[~m] > 0.0)
    assert abs(f.mean - f.kl[~m].sum() / (~m).sum()) < 1e-15
    full = d.forward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight)
    assert np.array_equal(full.kl[~m], f.kl[~m])
    dh, dw = d.backward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, x.labels)
    assert np.all(dh[m] == 0.0)
    keep = np.nonzero(~m)[0]
    dh2, dw2 = d.backward(x.s_hidden[keep], x.s_weight, x.t_hidden[keep], x.t_weight)
    assert np.allclose(dw, dw2, rtol=1e-12, atol=1e-15)
    assert np.allclose(dh[keep], dh2, rtol=1e-12, atol=1e-15)


def check_rows_helpers(d):
    x = _case(13, 8, 10, 50, seed=19, ignore_frac=0.2, reduction="none")
    tr = fo.LogitTransform(softcap=2.0, temperature=0.9)
    f = d.forward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, x.labels, transform=tr)
    rows = [0, 4, 12]
    kl, ls, lt = d.forward_rows(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, rows,
                                x.labels, transform=tr)
    assert np.allclose(kl, f.kl[rows], rtol=1e-13, atol=1e-15)
    assert np.allclose(ls, f.lse_s[rows]) and np.allclose(lt, f.lse_t[rows])
    c = d.token_scale(x.labels, 13, grad_out=x.grad_out)
    dh, dw = d.backward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, x.labels,
                        grad_out=x.grad_out, transform=tr)
    rh = d.grad_hidden_rows(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, rows, c[rows],
                            transform=tr)
    assert np.allclose(rh, dh[rows], rtol=1e-12, atol=1e-15)
    vr = [0, 7, 49]
    rw = d.grad_weight_rows(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, vr, c, f.lse_s,
                            f.lse_t, transform=tr)
    assert np.allclose(rw, dw[vr], rtol=1e-12, atol=1e-15)


def check_gradient_rows_sum_to_zero(d):
    x = _case(7, 8, 9, 33, seed=23)
    dh, dw = d.backward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight)
    col = np.abs(dw.sum(axis=0)).max()
    assert col < 1e-13 * max(1.0, np.abs(dw).max()), col


# --- generalized Jensen-Shannon divergence (divergence="jsd") ---

def check_jsd_identical_heads(d):
    x = _case(9, 16, 16, 37, seed=3)
    for beta in (0.5, 0.2):
        f = d.forward(x.s_hidden, x.s_weight, x.s_hidden, x.s_weight, divergence="jsd", beta=beta)
        assert np.max(np.abs(f.kl)) < 1e-13, f.kl
        dh, dw = d.backward(x.s_hidden, x.s_weight, x.s_hidden, x.s_weight, divergence="jsd",
                            beta=beta)
        assert np.max(np.abs(dh)) < 1e-14 and np.max(np.abs(dw)) < 1e-14


def check_jsd_symmetric_and_bounded(d):
    """beta = 1/2: symmetric in the two distributions and within [0, ln 2]; supports
    that barely overlap approach ln 2."""
    x = _case(6, 8, 8, 29, seed=41, ws=0.9, wt=0.9)
    a = d.forward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, divergence="jsd", beta=0.5)
    b = d.forward(x.t_hidden, x.t_weight, x.s_hidden, x.s_weight, divergence="jsd", beta=0.5)
    assert np.allclose(a.kl, b.kl, rtol=1e-12, atol=1e-15), (a.kl, b.kl)
    assert np.all(a.kl >= 0.0) and np.all(a.kl <= math.log(2.0) + 1e-15)
    T, V = 4, 40
    labels = np.array([3, 17, 0, 39], dtype=np.int64)
    th, tw = _onehot_teacher(T, T, V, labels)
    sh, sw = _onehot_teacher(T, T, V, (labels + 5) % V)
    f = d.forward(sh, sw, th, tw, divergence="jsd", beta=0.5)
    assert np.allclose(f.kl, math.log(2.0), rtol=0, atol=1e-12), f.kl


def check_jsd_limits_are_the_two_kls(d):
    """JSD_beta / beta -> KL(p_t || p_s) as beta -> 0, JSD_beta / (1 - beta) -> KL(p_s || p_t)
    as beta -> 1 (both KLs from the forward-KL path, pinned above)."""
    x = _case(5, 8, 9, 23, seed=43, ws=0.7, wt=0.7)
    fwd = d.forward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight).kl
    rev = d.forward(x.t_hidden, x.t_weight, x.s_hidden, x.s_weight).kl
    # JSD_b / b = KL + O(b): Richardson's 2 J(b)/b - J(2b)/(2b) removes the first-order term
    def ratio(b, near_one):
        beta = 1.0 - b if near_one else b
        return d.forward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, divergence="jsd",
                         beta=beta).kl / b

    eps = 1e-6
    lo = 2 * ratio(eps, False) - ratio(2 * eps, False)
    hi = 2 * ratio(eps, True) - ratio(2 * eps, True)
    assert np.allclose(lo, fwd, rtol=1e-6, atol=1e-10), (lo, fwd)
    assert np.allclose(hi, rev, rtol=1e-6, atol=1e-10), (hi, rev)


def check_jsd_two_class(d):
    T, Hs, Ht, V = 5, 8, 7, 2
    x = _case(T, Hs, Ht, V, seed=47, ws=1.0, wt=1.0)
    beta = 0.3
    f = d.forward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, divergence="jsd", beta=beta)
    hs = [py_decode(x.s_hidden[t]) for t in range(T)]
    ht = [py_decode(x.t_hidden[t]) for t in range(T)]
    ws = [py_decode(x.s_weight[v]) for v in range(V)]
    wt = [py_decode(x.t_weight[v]) for v in range(V)]
    for t in range(T):
        ds = math.fsum(a * b for a, b in zip(hs[t], ws[1])) - math.fsum(
            a * b for a, b in zip(hs[t], ws[0]))
        dt = math.fsum(a * b for a, b in zip(ht[t], wt[1])) - math.fsum(
            a * b for a, b in zip(ht[t], wt[0]))
        q1 = 1.0 / (1.0 + math.exp(-ds))
        p1 = 1.0 / (1.0 + math.exp(-dt))
        want = 0.0
        for p, q in ((p1, q1), (1 - p1, 1 - q1)):
            m = beta * p + (1 - beta) * q
            want += beta * p * math.log(p / m) + (1 - beta) * q * math.log(q / m)
        assert abs(f.kl[t] - want) < 1e-12, (t, f.kl[t], want)


def _fd_check_jsd(d, transform, beta):
    x = _case(5, 6, 7, 13, seed=53, ws=0.8, wt=0.8)
    hs, ws = fo.decode_bf16(x.s_hidden), fo.decode_bf16(x.s_weight)
    ht, wt = fo.decode_bf16(x.t_hidden), fo.decode_bf16(x.t_weight)
    labels = np.array([0, 0, IGN, 0, 0], dtype=np.int64)

    def loss(h, w):
        return d.forward(h, w, ht, wt, labels, transform=transform, divergence="jsd",
                         beta=beta).mean

    dh, dw = d.backward(hs, ws, ht, wt, labels, transform=transform, divergence="jsd", beta=beta)
    rng = np.random.default_rng(1)
    for arr, grad in ((hs, dh), (ws, dw)):
        for _ in range(12):
            i = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[i]
            arr[i] = old + 1e-6
            lp = loss(hs, ws)
            arr[i] = old - 1e-6
            lm = loss(hs, ws)
            arr[i] = old
            num = (lp - lm) / 2e-6
            assert abs(num - grad[i]) < 1e-8 + 1e-6 * abs(num), (i, num, grad[i])
    assert np.all(dh[2] == 0.0)


def check_jsd_finite_differences(d):
    _fd_check_jsd(d, None, 0.5)
    _fd_check_jsd(d, fo.LogitTransform(scale_multiply=1.3, softcap=1.5, temperature=0.7), 0.25)


def check_jsd_rows_helpers(d):
    x = _case(13, 8, 10, 50, seed=59, ignore_frac=0.2, reduction="none")
    tr = fo.LogitTransform(softcap=2.0, temperature=0.9)
    kw = dict(transform=tr, divergence="jsd", beta=0.35)
    f = d.forward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, x.labels, **kw)
    rows = [0, 4, 12]
    kl, _, _ = d.forward_rows(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, rows, x.labels,
                              **kw)
    assert np.allclose(kl, f.kl[rows], rtol=1e-13, atol=1e-15)
    c = d.token_scale(x.labels, 13, grad_out=x.grad_out)
    dh, dw = d.backward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, x.labels,
                        grad_out=x.grad_out, **kw)
    rh = d.grad_hidden_rows(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, rows, c[rows], **kw)
    assert np.allclose(rh, dh[rows], rtol=1e-12, atol=1e-15)
    gbar = d.jsd_gbar(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, beta=0.35, transform=tr)
    vr = [0, 7, 49]
    rw = d.grad_weight_rows(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, vr, c, f.lse_s,
                            f.lse_t, gbar=gbar, **kw)
    assert np.allclose(rw, dw[vr], rtol=1e-12, atol=1e-15)


def check_row_blocks(d):
    """Row blocks are a schedule detail: with one or two rows per block the divergence,
    both log-sum-exps, the student's gradients and the JSD row sums match the
    single-block results, and the brute-forced closed forms still hold."""
    with small_blocks(d.fo, 1):
        check_uniform_teacher(d)
        check_onehot_teacher_is_cross_entropy(d)
    T, Hs, Ht, V = 9, 8, 6, 17
    x = _case(T, Hs, Ht, V, seed=61, ignore_frac=0.2, reduction="none")
    args = (x.s_hidden, x.s_weight, x.t_hidden, x.t_weight)
    tr = fo.LogitTransform(softcap=2.5, temperature=0.9)
    for kw in (dict(divergence="kl"), dict(divergence="jsd", beta=0.3),
               dict(divergence="kl", transform=tr), dict(divergence="jsd", beta=0.6,
                                                         transform=tr)):
        f1 = d.forward(*args, x.labels, **kw)
        b1 = d.backward(*args, x.labels, grad_out=x.grad_out, **kw)
        gb1 = (d.jsd_gbar(*args, beta=kw["beta"], transform=kw.get("transform"))
               if kw["divergence"] == "jsd" else None)
        for elems in (1, 2 * V):
            with small_blocks(d.fo, elems):
                assert d.fo._rows_per_block(V, T) == max(1, elems // V)
                f2 = d.forward(*args, x.labels, **kw)
                b2 = d.backward(*args, x.labels, grad_out=x.grad_out, **kw)
                gb2 = (d.jsd_gbar(*args, beta=kw["beta"], transform=kw.get("transform"))
                       if gb1 is not None else None)
            for a, b in ((f2.kl, f1.kl), (f2.lse_s, f1.lse_s), (f2.lse_t, f1.lse_t),
                         (b2[0], b1[0]), (b2[1], b1[1])):
                assert np.allclose(a, b, rtol=1e-13, atol=1e-15), np.abs(a - b).max()
            assert abs(f2.mean - f1.mean) < 1e-13
            if gb1 is not None:
                assert np.allclose(gb2, gb1, rtol=1e-13, atol=1e-15)


ALL_CHECKS = [
    check_identical_heads,
    check_uniform_teacher,
    check_onehot_teacher_is_cross_entropy,
    check_two_class,
    check_finite_differences,
    check_finite_differences_transformed,
    check_mask_and_mean,
    check_rows_helpers,
    check_gradient_rows_sum_to_zero,
    check_jsd_identical_heads,
    check_jsd_symmetric_and_bounded,
    check_jsd_limits_are_the_two_kls,
    check_jsd_two_class,
    check_jsd_finite_differences,
    check_jsd_rows_helpers,
    check_row_blocks,
]
