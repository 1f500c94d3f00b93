"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

Each ``check_*`` takes the oracle module as an argument and raises
AssertionError when the oracle disagrees with an independent fact:

* closed forms (lm_head = 0 gives NLL = ln V; two classes give a softplus),
* brute force on tiny inputs with Python's ``math.fsum`` over exactly decoded
  bf16 values (no numpy matmul, no max shift),
* logits far beyond exp's float64 range must still give finite, exact answers,
* invariants (gradient rows of the logits sum to zero, so the vocabulary sum
  of dW is zero; ignored tokens contribute nothing; token order does not
  matter; log-prob = -NLL; the backward is linear in the upstream grad),
* central finite differences of the forward check the backward.

``test_oracle_mutants`` plants plausible mistakes in copies of the oracle and
requires that some check here fails for each of them.
"""
from __future__ import annotations

import contextlib
import math
import struct

import numpy as np

from chunked_lm_head_amd import synth

IGN = -100


def bf16_exact(values) -> np.ndarray:
    """uint16 bf16 bits of values that bf16 represents exactly (asserted)."""
    a = np.asarray(values, dtype=np.float64)
    f32 = a.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), a)
    u = f32.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def py_decode(bits) -> list:
    """bf16 bits -> Python floats through struct (independent of the oracle's decoder)."""
    return [struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in np.ravel(bits)]


def _rand_case(T, H, V, seed, w_std=0.5, ignore=()):
    w = synth.custom("pin", T=T, H=H, V=V, w_std=w_std, seed=seed)
    x = synth.make_inputs(w)
    labels = x.labels.copy()
    for t in ignore:
        labels[t] = IGN
    return x.hidden, x.weight, labels


def check_zero_weight(o):
    """lm_head = 0 => every logit is 0 => lse = NLL = ln V, log p = -ln V."""
    for T, H, V in [(5, 8, 7), (9, 16, 1000), (3, 8, 151936)]:
        h, _, labels = _rand_case(T, H, V, seed=T + V, ignore=(1,))
        w = np.zeros((V, H), dtype=np.uint16)
        f = o.forward(h, w, labels, IGN, "nll")
        valid = labels != IGN
        assert np.allclose(f.lse, math.log(V), rtol=1e-14, atol=0)
        assert np.allclose(f.out[valid], math.log(V), rtol=1e-14, atol=0)
        assert np.all(f.out[~valid] == 0.0)
        assert f.n_valid == T - 1
        assert abs(f.mean - math.log(V)) < 1e-12
        g = o.forward(h, w, labels, IGN, "logprob")
        assert np.allclose(g.out[valid], -math.log(V), rtol=1e-14, atol=0)
        assert abs(g.mean + math.log(V)) < 1e-12


def check_two_class(o):
    """T = 1, V = 2: NLL = softplus(z_other - z_label)."""
    h = bf16_exact([[1.0, 2.0]])
    w = bf16_exact([[0.5, 0.25], [-1.0, 3.0]])    # z = [1, 5]
    for label, other, mine in [(0, 5.0, 1.0), (1, 1.0, 5.0)]:
        f = o.forward(h, w, np.array([label]), IGN, "nll")
        expect = math.log1p(math.exp(other - mine))
        assert abs(f.out[0] - expect) < 1e-14, (f.out[0], expect)
        assert abs(f.lse[0] - (5.0 + math.log1p(math.exp(-4.0)))) < 1e-14


def _brute(hb, wb, labels, mode, grad_out, grad_mean):
    T, H = hb.shape
    V = wb.shape[0]
    h = np.array(py_decode(hb)).reshape(T, H).tolist()
    w = np.array(py_decode(wb)).reshape(V, H).tolist()
    z = [[math.fsum(h[t][k] * w[v][k] for k in range(H)) for v in range(V)] for t in range(T)]
    lse = [math.log(math.fsum(math.exp(z[t][v]) for v in range(V))) for t in range(T)]
    valid = [int(labels[t]) != IGN for t in range(T)]
    nvalid = sum(valid)
    out = []
    for t in range(T):
        if not valid[t]:
            out.append(0.0)
            continue
        nll = lse[t] - z[t][int(labels[t])]
        out.append(nll if mode == "nll" else -nll)
    mean = math.fsum(out) / nvalid if nvalid else 0.0
    c = []
    for t in range(T):
        if not valid[t]:
            c.append(0.0)
            continue
        g = float(grad_out[t]) if grad_out is not None else grad_mean / nvalid
        c.append(g if mode == "nll" else -g)
    G = [[c[t] * (math.exp(z[t][v] - lse[t]) - (1.0 if valid[t] and v == int(labels[t]) else 0.0))
          for v in range(V)] for t in range(T)]
    dh = [[math.fsum(G[t][v] * w[v][k] for v in range(V)) for k in range(H)] for t in range(T)]
    dw = [[math.fsum(G[t][v] * h[t][k] for t in range(T)) for k in range(H)] for v in range(V)]
    return np.array(out), np.array(lse), mean, np.array(dh), np.array(dw)


def check_bruteforce(o):
    """Tiny shapes against pure-Python sums over exactly decoded bf16 values."""
    cases = [
        (6, 5, 9, "nll", None, 1.0, (2,)),
        (4, 3, 7, "logprob", np.array([0.5, -1.25, 0.0, 2.0]), None, ()),
        (5, 8, 16, "nll", np.array([1.0, -0.5, 0.25, 3.0, -2.0]), None, (0, 4)),
        (3, 4, 5, "logprob", None, 0.75, (1,)),
    ]
    for i, (T, H, V, mode, g, gm, ign) in enumerate(cases):
        hb, wb, labels = _rand_case(T, H, V, seed=100 + i, w_std=0.7, ignore=ign)
        out, lse, mean, dh, dw = _brute(hb, wb, labels, mode, g, gm)
        f = o.forward(hb, wb, labels, IGN, mode)
        assert np.allclose(f.out, out, rtol=1e-12, atol=1e-12), (f.out, out)
        assert np.allclose(f.lse, lse, rtol=1e-12, atol=1e-12)
        assert abs(f.mean - mean) < 1e-12
        if g is not None:
            odh, odw = o.backward(hb, wb, labels, IGN, mode, grad_out=g)
        else:
            odh, odw = o.backward(hb, wb, labels, IGN, mode, grad_mean=gm)
        assert np.allclose(odh, dh, rtol=1e-11, atol=1e-13), np.abs(odh - dh).max()
        assert np.allclose(odw, dw, rtol=1e-11, atol=1e-13), np.abs(odw - dw).max()


def check_large_logits(o):
    """Logits of ~1000 overflow a naive exp in float64; the answer must stay exact."""
    h = bf16_exact([[64.0, 64.0], [64.0, 64.0]])
    w = bf16_exact([[8.0, 8.0], [8.0, 7.5], [0.0, 0.0]])   # z = [1024, 992, 0]
    with np.errstate(over="ignore", invalid="ignore"):
        f = o.forward(h, w, np.array([1, 0]), IGN, "nll")
        dh, dw = o.backward(h, w, np.array([1, 0]), IGN, "nll", grad_out=np.array([1.0, 1.0]))
    assert np.all(np.isfinite(f.out)) and np.all(np.isfinite(f.lse))
    assert abs(f.out[0] - (32.0 + math.log1p(math.exp(-32.0)))) < 1e-12
    assert abs(f.out[1] - math.log1p(math.exp(-32.0))) < 1e-12
    assert np.all(np.isfinite(dh)) and np.all(np.isfinite(dw))
    # token 0 (label 1): G = P - e_1 ~ (1, -1, 0); token 1 (label 0): G ~ (0, 0, 0)
    assert np.allclose(dh[0], [0.0, 0.5], atol=1e-9)


def check_ignore_index(o):
    """Ignored tokens: out = 0, zero dH row; removing them changes neither mean nor dW."""
    hb, wb, labels = _rand_case(11, 8, 13, seed=5, ignore=(0, 3, 10))
    f = o.forward(hb, wb, labels, IGN, "nll")
    dh, dw = o.backward(hb, wb, labels, IGN, "nll")
    ign = labels == IGN
    assert np.all(f.out[ign] == 0.0)
    assert np.all(dh[ign] == 0.0)
    keep = ~ign
    f2 = o.forward(hb[keep], wb, labels[keep], IGN, "nll")
    dh2, dw2 = o.backward(hb[keep], wb, labels[keep], IGN, "nll")
    assert abs(f.mean - f2.mean) < 1e-13
    assert np.allclose(dw, dw2, rtol=1e-12, atol=1e-14)
    assert np.allclose(dh[keep], dh2, rtol=1e-12, atol=1e-14)
    assert f.n_valid == keep.sum()


def check_vocab_sum_of_dw(o):
    """Each row of G sums to c_t (sum P - 1) = 0, so sum over vocab of dW is 0."""
    hb, wb, labels = _rand_case(17, 12, 29, seed=9, ignore=(2,))
    g = np.random.default_rng(3).standard_normal(17)
    for mode in ("nll", "logprob"):
        _, dw = o.backward(hb, wb, labels, IGN, mode, grad_out=g)
        scale = np.abs(dw).max()
        assert scale > 0
        assert np.abs(dw.sum(axis=0)).max() < 1e-12 * scale * 29


def check_zero_weight_backward(o):
    """lm_head = 0: dH = 0 and dW_v = sum_t c_t H_t / V - sum_{t: y_t = v} c_t H_t."""
    T, H, V = 7, 6, 5
    hb, _, labels = _rand_case(T, H, V, seed=11, ignore=(4,))
    w = np.zeros((V, H), dtype=np.uint16)
    g = np.array([0.5, -1.0, 2.0, 0.25, 3.0, -0.75, 1.5])
    dh, dw = o.backward(hb, w, labels, IGN, "nll", grad_out=g)
    assert np.all(dh == 0.0)
    h = np.array(py_decode(hb)).reshape(T, H)
    c = [g[t] if labels[t] != IGN else 0.0 for t in range(T)]
    for v in range(V):
        for k in range(H):
            expect = math.fsum(c[t] * h[t, k] / V for t in range(T)) - math.fsum(
                c[t] * h[t, k] for t in range(T) if labels[t] == v)
            assert abs(dw[v, k] - expect) < 1e-12, (v, k, dw[v, k], expect)


def _loss(o, h, w, labels, mode, g):
    f = o.forward(h, w, labels, IGN, mode)
    return float(np.dot(f.out, g)) if g is not None else f.mean


def check_finite_differences(o):
    """Central differences of the forward (float64 inputs) against the backward."""
    rng = np.random.default_rng(21)
    T, H, V = 5, 4, 7
    h = rng.standard_normal((T, H))
    w = rng.standard_normal((V, H)) * 0.8
    labels = np.array([3, IGN, 0, 6, 2])
    for mode, g in [("nll", None), ("nll", rng.standard_normal(T)),
                    ("logprob", rng.standard_normal(T))]:
        if g is None:
            dh, dw = o.backward(h, w, labels, IGN, mode, grad_mean=1.0)
        else:
            dh, dw = o.backward(h, w, labels, IGN, mode, grad_out=g)
        eps = 1e-6
        for arr, grad in ((h, dh), (w, dw)):
            num = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                keep = arr[idx]
                arr[idx] = keep + eps
                lp = _loss(o, h, w, labels, mode, g)
                arr[idx] = keep - eps
                lm = _loss(o, h, w, labels, mode, g)
                arr[idx] = keep
                num[idx] = (lp - lm) / (2 * eps)
            assert np.allclose(grad, num, rtol=1e-6, atol=1e-8), np.abs(grad - num).max()


def check_duality_and_linearity(o):
    """log p = -NLL; backward(logprob, g) = backward(nll, -g); linear in g; g = 0 gives 0."""
    hb, wb, labels = _rand_case(9, 8, 11, seed=31, ignore=(5,))
    a = o.forward(hb, wb, labels, IGN, "nll")
    b = o.forward(hb, wb, labels, IGN, "logprob")
    assert np.array_equal(a.out, -b.out)
    rng = np.random.default_rng(2)
    g1, g2 = rng.standard_normal(9), rng.standard_normal(9)
    d_lp = o.backward(hb, wb, labels, IGN, "logprob", grad_out=g1)
    d_nl = o.backward(hb, wb, labels, IGN, "nll", grad_out=-g1)
    for x, y in zip(d_lp, d_nl):
        assert np.allclose(x, y, rtol=1e-13, atol=1e-15)
    s = o.backward(hb, wb, labels, IGN, "nll", grad_out=2.0 * g1 - 3.0 * g2)
    p = o.backward(hb, wb, labels, IGN, "nll", grad_out=g1)
    q = o.backward(hb, wb, labels, IGN, "nll", grad_out=g2)
    for x, y, zz in zip(s, p, q):
        assert np.allclose(x, 2.0 * y - 3.0 * zz, rtol=1e-11, atol=1e-13)
    zero = o.backward(hb, wb, labels, IGN, "nll", grad_out=np.zeros(9))
    assert all(np.all(x == 0.0) for x in zero)
    # mean reduction = per-token grad of 1/n_valid on every used token
    n = int((labels != IGN).sum())
    m = o.backward(hb, wb, labels, IGN, "nll", grad_mean=1.0)
    t = o.backward(hb, wb, labels, IGN, "nll", grad_out=np.full(9, 1.0 / n))
    for x, y in zip(m, t):
        assert np.allclose(x, y, rtol=1e-13, atol=1e-15)


def check_token_permutation(o):
    """Permuting tokens permutes out and dH and leaves dW and the mean unchanged."""
    hb, wb, labels = _rand_case(10, 8, 12, seed=41, ignore=(7,))
    perm = np.random.default_rng(4).permutation(10)
    f = o.forward(hb, wb, labels, IGN, "nll")
    fp = o.forward(hb[perm], wb, labels[perm], IGN, "nll")
    assert np.allclose(fp.out, f.out[perm], rtol=1e-14, atol=1e-15)
    assert abs(fp.mean - f.mean) < 1e-13
    dh, dw = o.backward(hb, wb, labels, IGN, "nll")
    dhp, dwp = o.backward(hb[perm], wb, labels[perm], IGN, "nll")
    assert np.allclose(dhp, dh[perm], rtol=1e-13, atol=1e-15)
    assert np.allclose(dwp, dw, rtol=1e-12, atol=1e-15)


def check_row_helpers(o):
    """The sampled-row helpers agree with the full forward/backward."""
    hb, wb, labels = _rand_case(13, 8, 21, seed=51, ignore=(6,))
    g = np.random.default_rng(5).standard_normal(13)
    f = o.forward(hb, wb, labels, IGN, "logprob")
    dh, dw = o.backward(hb, wb, labels, IGN, "logprob", grad_out=g)
    rows = [0, 6, 12]
    out, lse = o.forward_rows(hb, wb, labels, rows, IGN, "logprob")
    assert np.allclose(out, f.out[rows], rtol=1e-13, atol=1e-15)
    assert np.allclose(lse, f.lse[rows], rtol=1e-13, atol=1e-15)
    c = o.token_scale(labels, 21, IGN, "logprob", grad_out=g)
    assert np.allclose(o.grad_hidden_rows(hb, wb, labels, rows, c[rows], IGN), dh[rows],
                       rtol=1e-12, atol=1e-14)
    vr = [0, 5, 20, int(labels[0])]
    assert np.allclose(o.grad_weight_rows(hb, wb, labels, vr, c, f.lse), dw[vr],
                       rtol=1e-12, atol=1e-14)


def check_out_of_range_label_raises(o):
    hb, wb, labels = _rand_case(4, 8, 6, seed=61)
    labels[2] = 6
    try:
        o.forward(hb, wb, labels, IGN, "nll")
    except ValueError:
        return
    raise AssertionError("out-of-range label was accepted")


# --- logit transforms (Unsloth page, section "Chunking der abgeflachten Sequenzlaenge": the
# chunked call's logit_scale_multiply / logit_scale_divide / logit_softcapping / temperature) ---


def check_transform_linear(o):
    """Without softcap the transform is one positive scale s = mul / div / temperature, so it
    must equal the untransformed oracle on s W (exact in bf16 for powers of two), with
    dH unchanged and dW scaled by s (chain rule through W' = s W)."""
    hb, wb, labels = _rand_case(7, 8, 13, seed=71, w_std=0.6, ignore=(3,))
    g = np.linspace(-1.0, 2.0, 7)
    w64 = o.decode_bf16(wb)
    for tf, s in [(o.LogitTransform(temperature=2.0), 0.5),
                  (o.LogitTransform(scale_multiply=4.0, scale_divide=2.0), 2.0),
                  (o.LogitTransform(scale_multiply=0.5, temperature=0.25), 2.0),
                  (o.LogitTransform(scale_divide=8.0), 0.125)]:
        ws = bf16_exact(w64 * s)
        for mode in ("nll", "logprob"):
            a = o.forward(hb, wb, labels, IGN, mode, transform=tf)
            b = o.forward(hb, ws, labels, IGN, mode)
            assert np.allclose(a.out, b.out, rtol=1e-13, atol=1e-13), (tf, a.out, b.out)
            assert np.allclose(a.lse, b.lse, rtol=1e-13, atol=1e-13)
            dha, dwa = o.backward(hb, wb, labels, IGN, mode, grad_out=g, transform=tf)
            dhb, dwb = o.backward(hb, ws, labels, IGN, mode, grad_out=g)
            assert np.allclose(dha, dhb, rtol=1e-12, atol=1e-14), np.abs(dha - dhb).max()
            assert np.allclose(dwa, s * dwb, rtol=1e-12, atol=1e-14), np.abs(dwa - s * dwb).max()
    # a scale that is not a power of two, on float64 inputs
    h64 = o.decode_bf16(hb)
    a = o.forward(h64, w64, labels, IGN, "nll", transform=o.LogitTransform(scale_multiply=3.0))
    b = o.forward(h64, 3.0 * w64, labels, IGN, "nll")
    assert np.allclose(a.out, b.out, rtol=1e-12, atol=1e-12)


def check_softcap_saturation(o):
    """Logits far beyond the cap saturate tanh to exactly +-1 in float64, so every transformed
    logit is +-cap / temperature and lse = ln(k e^c + (V - k) e^-c) with c = cap / temperature
    and k the number of positive logits: a closed form that also fixes the order (scaling
    before the cap, temperature after it)."""
    T, H, V = 4, 2, 9
    h = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-1.0, 0.5]])
    w = np.array([[3e3 * (1 if (v % 3) else -1), 2e3 * (1 if v % 2 else -1)] for v in range(V)])
    labels = np.array([0, 1, 4, 7])
    z = h @ w.T
    assert np.all(np.abs(z) > 400.0)
    for cap, temp, mul in [(10.0, 1.0, 0.0), (10.0, 2.0, 0.0), (5.0, 0.5, 4.0), (30.0, 3.0, 0.5)]:
        tf = o.LogitTransform(scale_multiply=mul, softcap=cap, temperature=temp)
        f = o.forward(h, w, labels, IGN, "nll", transform=tf)
        c = cap / temp
        for t in range(T):
            k = int((z[t] > 0).sum())
            lse = math.log(k * math.exp(c) + (V - k) * math.exp(-c))
            zy = c if z[t, labels[t]] > 0 else -c
            assert abs(f.lse[t] - lse) < 1e-12, (tf, t, f.lse[t], lse)
            assert abs(f.out[t] - (lse - zy)) < 1e-12
    # a tiny scale before the cap keeps the logits far from it: no saturation at all
    tf = o.LogitTransform(scale_multiply=1e-6, softcap=10.0)
    f = o.forward(h, w, labels, IGN, "nll", transform=tf)
    g = o.forward(h, w * 1e-6, labels, IGN, "nll")
    assert np.allclose(f.out, g.out, rtol=1e-6, atol=1e-9)


def check_softcap_limits(o):
    """A cap far above every logit changes nothing; the softcap is odd in the logits."""
    hb, wb, labels = _rand_case(6, 8, 11, seed=81, w_std=0.6)
    a = o.forward(hb, wb, labels, IGN, "nll", transform=o.LogitTransform(softcap=1e9))
    b = o.forward(hb, wb, labels, IGN, "nll")
    assert np.allclose(a.out, b.out, rtol=1e-12, atol=1e-12)
    h64, w64 = o.decode_bf16(hb), o.decode_bf16(wb)
    tf = o.LogitTransform(softcap=1.5, temperature=0.7)
    zp, dp = tf.apply(h64 @ w64.T)
    zm, dm = tf.apply(h64 @ (-w64).T)
    assert np.allclose(zp, -zm, rtol=0, atol=1e-15) and np.allclose(dp, dm, rtol=0, atol=1e-15)
    assert np.all(np.abs(zp) < 1.5 / 0.7)


def _tloss(o, h, w, labels, mode, g, tf):
    f = o.forward(h, w, labels, IGN, mode, transform=tf)
    return float(np.dot(f.out, g)) if g is not None else f.mean


def check_transform_finite_differences(o):
    """Central differences of the transformed forward against the backward's chain rule."""
    rng = np.random.default_rng(91)
    T, H, V = 4, 3, 6
    h = rng.standard_normal((T, H)) * 1.5
    w = rng.standard_normal((V, H)) * 1.2
    labels = np.array([2, 0, IGN, 5])
    for tf, mode, g in [
            (o.LogitTransform(softcap=1.5), "nll", None),
            (o.LogitTransform(scale_multiply=2.0, softcap=2.0, temperature=0.8), "nll",
             rng.standard_normal(T)),
            (o.LogitTransform(scale_divide=3.0, temperature=1.7), "logprob", rng.standard_normal(T)),
            (o.LogitTransform(scale_multiply=0.7, scale_divide=0.9, softcap=0.6, temperature=1.3),
             "logprob", rng.standard_normal(T))]:
        if g is None:
            dh, dw = o.backward(h, w, labels, IGN, mode, grad_mean=1.0, transform=tf)
        else:
            dh, dw = o.backward(h, w, labels, IGN, mode, grad_out=g, transform=tf)
        eps = 1e-6
        for arr, grad in ((h, dh), (w, dw)):
            num = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                keep = arr[idx]
                arr[idx] = keep + eps
                lp = _tloss(o, h, w, labels, mode, g, tf)
                arr[idx] = keep - eps
                lm = _tloss(o, h, w, labels, mode, g, tf)
                arr[idx] = keep
                num[idx] = (lp - lm) / (2 * eps)
            assert np.allclose(grad, num, rtol=1e-6, atol=1e-8), (tf, np.abs(grad - num).max())


def check_transform_rows_and_args(o):
    """Row helpers agree with the full computation under a transform; invalid values raise."""
    hb, wb, labels = _rand_case(8, 8, 10, seed=95, w_std=0.6, ignore=(6,))
    tf = o.LogitTransform(scale_multiply=1.5, softcap=2.0, temperature=0.9)
    g = np.linspace(-1.0, 1.0, 8)
    f = o.forward(hb, wb, labels, IGN, "nll", transform=tf)
    dh, dw = o.backward(hb, wb, labels, IGN, "nll", grad_out=g, transform=tf)
    rows = [0, 3, 7]
    out_r, lse_r = o.forward_rows(hb, wb, labels, rows, IGN, "nll", transform=tf)
    assert np.allclose(out_r, f.out[rows], rtol=1e-13, atol=1e-13)
    assert np.allclose(lse_r, f.lse[rows], rtol=1e-13, atol=1e-13)
    c = o.token_scale(labels, 10, IGN, "nll", grad_out=g)
    dhr = o.grad_hidden_rows(hb, wb, labels, rows, c[rows], IGN, transform=tf)
    assert np.allclose(dhr, dh[rows], rtol=1e-12, atol=1e-14)
    dwr = o.grad_weight_rows(hb, wb, labels, [1, 4, 9], c, f.lse, transform=tf)
    assert np.allclose(dwr, dw[[1, 4, 9]], rtol=1e-12, atol=1e-14)
    for bad in (dict(temperature=0.0), dict(temperature=-1.0), dict(softcap=-1.0),
                dict(scale_multiply=-2.0), dict(scale_divide=-0.5)):
        try:
            o.forward(hb, wb, labels, IGN, "nll", transform=o.LogitTransform(**bad))
        except ValueError:
            continue
        raise AssertionError(f"invalid transform {bad} was accepted")


@contextlib.contextmanager
def small_blocks(o, elems):
    """The oracle's row blocks forced down to ``elems`` logits each, so that every call
    below runs its row-blocked loop over several blocks (at least one row per block)."""
    saved = o._BLOCK_ELEMS
    o._BLOCK_ELEMS = elems
    try:
        yield
    finally:
        o._BLOCK_ELEMS = saved


def check_row_blocks(o):
    """Row blocks are a schedule detail: with one or three rows per block the results
    match the brute force and the single-block results.  The full-size expected values
    are generated through many blocks, so this is their pin."""
    with small_blocks(o, 1):
        check_bruteforce(o)                  # independent facts, one row per block
        check_ignore_index(o)
    T, H, V = 11, 8, 13
    hb, wb, labels = _rand_case(T, H, V, seed=77, w_std=0.6, ignore=(2, 9))
    g = np.random.default_rng(77).standard_normal(T)
    tf = o.LogitTransform(scale_multiply=1.5, softcap=3.0, temperature=0.8)
    for mode in ("nll", "logprob"):
        for tr in (None, tf):
            f1 = o.forward(hb, wb, labels, IGN, mode, transform=tr)
            b1 = o.backward(hb, wb, labels, IGN, mode, grad_out=g, transform=tr)
            m1 = o.backward(hb, wb, labels, IGN, mode, grad_mean=0.7, lse=f1.lse, transform=tr)
            for elems in (1, 3 * V):         # 1 row, then 3 rows (ragged last block)
                with small_blocks(o, elems):
                    assert o._rows_per_block(V, T) == max(1, elems // V)
                    f2 = o.forward(hb, wb, labels, IGN, mode, transform=tr)
                    b2 = o.backward(hb, wb, labels, IGN, mode, grad_out=g, transform=tr)
                    m2 = o.backward(hb, wb, labels, IGN, mode, grad_mean=0.7, lse=f2.lse,
                                    transform=tr)
                assert np.allclose(f2.out, f1.out, rtol=1e-13, atol=1e-15)
                assert np.allclose(f2.lse, f1.lse, rtol=1e-13, atol=1e-15)
                assert abs(f2.mean - f1.mean) < 1e-13
                for a, b in zip(b2 + m2, b1 + m1):
                    assert np.allclose(a, b, rtol=1e-13, atol=1e-15), np.abs(a - b).max()


def check_default_multiplier(o):
    """The page's default chunk multiplier max(4, context // 4096), evaluated by hand
    above the floor of 4, where a wrong divisor would show."""
    hand = {1: 4, 4096: 4, 8192: 4, 16383: 4, 16384: 4, 20480: 5, 24576: 6, 65536: 16,
            131072: 32, 1048576: 256}
    for ctx, mult in hand.items():
        assert o.default_multiplier(ctx) == mult, (ctx, o.default_multiplier(ctx), mult)


ALL_CHECKS = [
    check_zero_weight,
    check_two_class,
    check_bruteforce,
    check_large_logits,
    check_ignore_index,
    check_vocab_sum_of_dw,
    check_zero_weight_backward,
    check_finite_differences,
    check_duality_and_linearity,
    check_token_permutation,
    check_row_helpers,
    check_out_of_range_label_raises,
    check_transform_linear,
    check_softcap_saturation,
    check_softcap_limits,
    check_transform_finite_differences,
    check_transform_rows_and_args,
    check_row_blocks,
    check_default_multiplier,
]
