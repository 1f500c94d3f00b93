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


def forward(s_hidden, s_weight, t_hidden, t_weight, labels=None,
            ignore_index: int = IGNORE_INDEX,
            transform: Optional[fo.LogitTransform] = None) -> DistillForward:
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
        kl[r0:r1] = (np.exp(log_pt) * (log_pt - log_ps)).sum(axis=1)
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


def grad_logits(zs, zt, c, dzs=None) -> np.ndarray:
    """G = c_t (softmax(zs_t) - softmax(zt_t)), times dzs'/dzs under a transform."""
    g = (np.exp(_log_softmax(zs)) - np.exp(_log_softmax(zt))) * c[:, None]
    return g if dzs is None else g * dzs


def backward(s_hidden, s_weight, t_hidden, t_weight, labels=None,
             ignore_index: int = IGNORE_INDEX, grad_out: Optional[np.ndarray] = None,
             grad_mean: Optional[float] = None,
             transform: Optional[fo.LogitTransform] = None):
    """(dHs [T, Hs], dWs [V, Hs]) in float64; the teacher receives no gradient."""
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
        g = grad_logits(zs, zt, c[r0:r1], dzs)
        dh[r0:r1] = g @ ws
        dw += g.T @ hs[r0:r1]
    return dh, dw


def forward_rows(s_hidden, s_weight, t_hidden, t_weight, rows: Sequence[int], labels=None,
                 ignore_index: int = IGNORE_INDEX,
                 transform: Optional[fo.LogitTransform] = None):
    """(kl, lse_s, lse_t) of the selected tokens only (each row needs its own logits)."""
    rows = np.asarray(rows, dtype=np.int64)
    lab = None if labels is None else np.asarray(labels)[rows]
    f = forward(np.asarray(s_hidden)[rows], s_weight, np.asarray(t_hidden)[rows], t_weight,
                lab, ignore_index, transform)
    return f.kl, f.lse_s, f.lse_t


def grad_hidden_rows(s_hidden, s_weight, t_hidden, t_weight, rows: Sequence[int],
                     c_rows: np.ndarray, transform: Optional[fo.LogitTransform] = None):
    """dHs rows of the selected tokens given their scales c_t."""
    rows = np.asarray(rows, dtype=np.int64)
    hs, ws = fo._as_f64(np.asarray(s_hidden)[rows]), fo._as_f64(s_weight)
    ht, wt = fo._as_f64(np.asarray(t_hidden)[rows]), fo._as_f64(t_weight)
    zs, dzs = fo._logits(hs, ws, transform)
    zt, _ = fo._logits(ht, wt, transform)
    return grad_logits(zs, zt, np.asarray(c_rows, dtype=np.float64), dzs) @ ws


def grad_weight_rows(s_hidden, s_weight, t_hidden, t_weight, vocab_rows: Sequence[int],
                     c: np.ndarray, lse_s: np.ndarray, lse_t: np.ndarray,
                     transform: Optional[fo.LogitTransform] = None) -> np.ndarray:
    """dWs rows of the selected vocabulary entries: dWs_v = sum_t G_tv hs_t.

    Needs both log-sum-exps of every token (from ``forward``); only the
    selected columns of the logits are formed."""
    vr = np.asarray(vocab_rows, dtype=np.int64)
    hs = fo._as_f64(s_hidden)
    ht = fo._as_f64(t_hidden)
    zs, dzs = fo._logits(hs, fo._as_f64(np.asarray(s_weight)[vr]), transform)
    zt, _ = fo._logits(ht, fo._as_f64(np.asarray(t_weight)[vr]), transform)
    g = np.exp(zs - np.asarray(lse_s)[:, None]) - np.exp(zt - np.asarray(lse_t)[:, None])
    g *= np.asarray(c, dtype=np.float64)[:, None]
    if dzs is not None:
        g *= dzs
    return g.T @ hs
