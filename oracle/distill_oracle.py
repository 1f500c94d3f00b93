"""CPU oracle for chunked distillation through two LM heads (student, teacher).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module; the product path never does.
It shares no code with the HIP library and imports nothing from it.

Source: TRL v1.13 article, speed section: the bf16 fix of the chunked loss is
applied to the distillation trainer too, which computes every chunk twice,
once with the student's hidden states and lm_head and once with the
teacher's.  The pages name no divergence (the same article lists a fused
linear JSD loss among the losses moved into TRL, without a definition).

Reading (a plain, slow, obviously correct definition in float64):

* per token t, student logits ``zs = Ws hs_t`` and teacher logits
  ``zt = Wt ht_t`` over one vocabulary, each through the same optional logit
  transform as the cross-entropy path (``flce_oracle.LogitTransform``);
* ``ps = softmax(zs)``, ``pt = softmax(zt)`` and the per-token loss is the
  forward Kullback-Leibler divergence of the student from the teacher,
  ``KL_t = sum_v pt_v (log pt_v - log ps_v)``, the textbook distillation loss
  (the teacher's distribution is the target);
* tokens whose mask label equals ``ignore_index`` output 0, get no gradient
  and are left out of the mean (no labels: every token counts);
* only the student receives gradients: with the upstream scale c_t,
  ``dL/dzs = c_t (ps - pt)`` (times dzs'/dzs under a transform), so
  ``dHs = G Ws`` and ``dWs = G^T Hs``, exactly the cross-entropy backward
  with the one-hot target replaced by the teacher's distribution.

The same article lists a fused linear JSD loss by name.  ``divergence="jsd"``
takes the generalized Jensen-Shannon divergence with weight beta in (0, 1), the
textbook definition (Lin, 1991; the skewed form used for distillation):
``M = beta p_t + (1 - beta) p_s`` and
``JSD_t = beta KL(p_t || M) + (1 - beta) KL(p_s || M)`` (beta = 1/2 is the
symmetric JSD).  Its gradient in the student's logits is
``dJSD/dzs_v = p_s,v (g_v - sum_u p_s,u g_u)``, ``g = (1 - beta) log(p_s / M)``.

Large inputs are processed in row blocks of complete vocabulary rows; a block
is a schedule detail, not part of the method.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

from oracle import flce_oracle as fo

IGNORE_INDEX = fo.IGNORE_INDEX


def _mask(labels, T: int, ignore_index: int) -> np.ndarray:
    if labels is None:
        return np.ones(T, dtype=bool)
    return np.asarray(labels, dtype=np.int64) != ignore_index


def _log_softmax(z: np.ndarray) -> np.ndarray:
    return z - fo.logsumexp_rows(z)[:, None]


@dataclasses.dataclass
class DistillForward:
    kl: np.ndarray      # [T] per-token KL(teacher || student), 0 where masked
    lse_s: np.ndarray   # [T] log-sum-exp of the student's logit row
    lse_t: np.ndarray   # [T] log-sum-exp of the teacher's logit row
    mean: float         # sum of kl over used tokens / their number (0 if none)
    n_valid: int


def _rows(h, w, transform, r0, r1):
    return fo._logits(h[r0:r1], w, transform)


def _xlogy_ratio(a, log_a, log_m):
    """a (log a - log m), taken as 0 where a = 0."""
    return np.where(a > 0, a * (log_a - log_m), 0.0)


def jsd_rows(log_ps, log_pt, beta: float) -> np.ndarray:
    """Per-row generalized JSD of the student (log_ps) and teacher (log_pt) rows."""
    ps, pt = np.exp(log_ps), np.exp(log_pt)
    m = beta * pt + (1.0 - beta) * ps
    with np.errstate(divide="ignore"):
        log_m = np.log(m)
    return (beta * _xlogy_ratio(pt, log_pt, log_m)
            + (1.0 - beta) * _xlogy_ratio(ps, log_ps, log_m)).sum(axis=1)


def _check_divergence(divergence: str, beta: float) -> None:
    if divergence not in ("kl", "jsd"):
        raise ValueError(divergence)
    if divergence == "jsd" and not 0.0 < beta < 1.0:
        raise ValueError(f"beta = {beta} must lie in (0, 1)")


def forward(s_hidden, s_weight, t_hidden, t_weight, labels=None,
            ignore_index: int = IGNORE_INDEX,
            transform: Optional[fo.LogitTransform] = None, divergence: str = "kl",
            beta: float = 0.5) -> DistillForward:
    _check_divergence(divergence, beta)
    hs, ws = fo._as_f64(s_hidden), fo._as_f64(s_weight)
    ht, wt = fo._as_f64(t_hidden), fo._as_f64(t_weight)
    T, V = hs.shape[0], ws.shape[0]
    if wt.shape[0] != V or ht.shape[0] != T:
        raise ValueError("student and teacher must share tokens and vocabulary")
    valid = _mask(labels, T, ignore_index)
    kl = np.zeros(T)
    lse_s = np.empty(T)
    lse_t = np.empty(T)
    step = fo._rows_per_block(V, T)
    for r0 in range(0, T, step):
        r1 = min(T, r0 + step)
        zs, _ = _rows(hs, ws, transform, r0, r1)
        zt, _ = _rows(ht, wt, transform, r0, r1)
        lse_s[r0:r1] = fo.logsumexp_rows(zs)
        lse_t[r0:r1] = fo.logsumexp_rows(zt)
        log_ps = zs - lse_s[r0:r1, None]
        log_pt = zt - lse_t[r0:r1, None]
        if divergence == "kl":
            kl[r0:r1] = (np.exp(log_pt) * (log_pt - log_ps)).sum(axis=1)
        else:
            kl[r0:r1] = jsd_rows(log_ps, log_pt, beta)
    kl = np.where(valid, kl, 0.0)
    n_valid = int(valid.sum())
    mean = float(kl[valid].sum() / n_valid) if n_valid else 0.0
    return DistillForward(kl=kl, lse_s=lse_s, lse_t=lse_t, mean=mean, n_valid=n_valid)


def token_scale(labels, T: int, ignore_index: int = IGNORE_INDEX,
                grad_out: Optional[np.ndarray] = None,
                grad_mean: Optional[float] = None) -> np.ndarray:
    """c_t: dL/d kl_t per token (``grad_out``), or grad_mean / n_valid (default 1)."""
    valid = _mask(labels, T, ignore_index)
    if grad_out is not None:
        g = np.asarray(grad_out, dtype=np.float64).copy()
    else:
        n_valid = int(valid.sum())
        gm = 1.0 if grad_mean is None else float(grad_mean)
        g = np.full(T, gm / n_valid if n_valid else 0.0)
    return np.where(valid, g, 0.0)


def grad_logits(zs, zt, c, dzs=None, divergence: str = "kl", beta: float = 0.5) -> np.ndarray:
    """dL/dzs: KL: c_t (softmax(zs_t) - softmax(zt_t)); JSD: c_t p_s (g - sum p_s g) with
    g = (1 - beta) log(p_s / M); times dzs'/dzs under a transform."""
    if divergence == "kl":
        g = (np.exp(_log_softmax(zs)) - np.exp(_log_softmax(zt))) * c[:, None]
    else:
        log_ps, log_pt = _log_softmax(zs), _log_softmax(zt)
        ps = np.exp(log_ps)
        log_m = np.log(beta * np.exp(log_pt) + (1.0 - beta) * ps)
        gv = (1.0 - beta) * (log_ps - log_m)
        gbar = (ps * gv).sum(axis=1, keepdims=True)
        g = ps * (gv - gbar) * c[:, None]
    return g if dzs is None else g * dzs


def backward(s_hidden, s_weight, t_hidden, t_weight, labels=None,
             ignore_index: int = IGNORE_INDEX, grad_out: Optional[np.ndarray] = None,
             grad_mean: Optional[float] = None,
             transform: Optional[fo.LogitTransform] = None, divergence: str = "kl",
             beta: float = 0.5):
    """(dHs [T, Hs], dWs [V, Hs]) in float64; the teacher receives no gradient."""
    _check_divergence(divergence, beta)
    hs, ws = fo._as_f64(s_hidden), fo._as_f64(s_weight)
    ht, wt = fo._as_f64(t_hidden), fo._as_f64(t_weight)
    T, V = hs.shape[0], ws.shape[0]
    c = token_scale(labels, T, ignore_index, grad_out, grad_mean)
    dh = np.zeros_like(hs)
    dw = np.zeros_like(ws)
    step = fo._rows_per_block(V, T)
    for r0 in range(0, T, step):
        r1 = min(T, r0 + step)
        zs, dzs = _rows(hs, ws, transform, r0, r1)
        zt, _ = _rows(ht, wt, transform, r0, r1)
        g = grad_logits(zs, zt, c[r0:r1], dzs, divergence, beta)
        dh[r0:r1] = g @ ws
        dw += g.T @ hs[r0:r1]
    return dh, dw


def forward_rows(s_hidden, s_weight, t_hidden, t_weight, rows: Sequence[int], labels=None,
                 ignore_index: int = IGNORE_INDEX,
                 transform: Optional[fo.LogitTransform] = None, divergence: str = "kl",
                 beta: float = 0.5):
    """(kl, lse_s, lse_t) of the selected tokens only (each row needs its own logits)."""
    rows = np.asarray(rows, dtype=np.int64)
    lab = None if labels is None else np.asarray(labels)[rows]
    f = forward(np.asarray(s_hidden)[rows], s_weight, np.asarray(t_hidden)[rows], t_weight,
                lab, ignore_index, transform, divergence, beta)
    return f.kl, f.lse_s, f.lse_t


def grad_hidden_rows(s_hidden, s_weight, t_hidden, t_weight, rows: Sequence[int],
                     c_rows: np.ndarray, transform: Optional[fo.LogitTransform] = None,
                     divergence: str = "kl", beta: float = 0.5):
    """dHs rows of the selected tokens given their scales c_t."""
    rows = np.asarray(rows, dtype=np.int64)
    hs, ws = fo._as_f64(np.asarray(s_hidden)[rows]), fo._as_f64(s_weight)
    ht, wt = fo._as_f64(np.asarray(t_hidden)[rows]), fo._as_f64(t_weight)
    zs, dzs = fo._logits(hs, ws, transform)
    zt, _ = fo._logits(ht, wt, transform)
    return grad_logits(zs, zt, np.asarray(c_rows, dtype=np.float64), dzs, divergence, beta) @ ws


def grad_weight_rows(s_hidden, s_weight, t_hidden, t_weight, vocab_rows: Sequence[int],
                     c: np.ndarray, lse_s: np.ndarray, lse_t: np.ndarray,
                     transform: Optional[fo.LogitTransform] = None, divergence: str = "kl",
                     beta: float = 0.5, gbar: Optional[np.ndarray] = None) -> np.ndarray:
    """dWs rows of the selected vocabulary entries: dWs_v = sum_t G_tv hs_t.

    Needs both log-sum-exps of every token (from ``forward``), and for JSD the
    per-token sum_u p_s,u g_u (``jsd_gbar``); only the selected columns of the
    logits are formed."""
    vr = np.asarray(vocab_rows, dtype=np.int64)
    hs = fo._as_f64(s_hidden)
    ht = fo._as_f64(t_hidden)
    zs, dzs = fo._logits(hs, fo._as_f64(np.asarray(s_weight)[vr]), transform)
    zt, _ = fo._logits(ht, fo._as_f64(np.asarray(t_weight)[vr]), transform)
    log_ps = zs - np.asarray(lse_s)[:, None]
    log_pt = zt - np.asarray(lse_t)[:, None]
    if divergence == "kl":
        g = np.exp(log_ps) - np.exp(log_pt)
    else:
        ps = np.exp(log_ps)
        gv = (1.0 - beta) * (log_ps - np.log(beta * np.exp(log_pt) + (1.0 - beta) * ps))
        g = ps * (gv - np.asarray(gbar)[:, None])
    g *= np.asarray(c, dtype=np.float64)[:, None]
    if dzs is not None:
        g *= dzs
    return g.T @ hs


def jsd_gbar(s_hidden, s_weight, t_hidden, t_weight, beta: float = 0.5,
             transform: Optional[fo.LogitTransform] = None) -> np.ndarray:
    """Per token sum_v p_s,v g_v, g = (1 - beta) log(p_s / M): the row sum the JSD
    gradient subtracts (full vocabulary rows)."""
    hs, ws = fo._as_f64(s_hidden), fo._as_f64(s_weight)
    ht, wt = fo._as_f64(t_hidden), fo._as_f64(t_weight)
    T, V = hs.shape[0], ws.shape[0]
    out = np.empty(T)
    step = fo._rows_per_block(V, T)
    for r0 in range(0, T, step):
        r1 = min(T, r0 + step)
        zs, _ = _rows(hs, ws, transform, r0, r1)
        zt, _ = _rows(ht, wt, transform, r0, r1)
        log_ps, log_pt = _log_softmax(zs), _log_softmax(zt)
        ps = np.exp(log_ps)
        gv = (1.0 - beta) * (log_ps - np.log(beta * np.exp(log_pt) + (1.0 - beta) * ps))
        out[r0:r1] = (ps * gv).sum(axis=1)
    return out
