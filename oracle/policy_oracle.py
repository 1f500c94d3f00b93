"""CPU oracle for policy-optimisation losses on top of the chunked selective log-softmax.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module; the product path never does.
It shares no code with the HIP library and imports nothing from it.

Source on the pages: the TRL v1.13 article, section on the other v1.13 changes
(fused losses folded into ``trl.losses``), names fused linear GRPO, DPO and KTO
losses built on the chunked LM head; the Unsloth GRPO long-context page feeds
the chunked selective log-softmax (per-token log p of the completion ids) into
GRPO.  Neither page defines the losses, so this oracle writes out the published
definitions (a reading; each is listed with its reason in the design notes):

* per-token log-probs ``logp_t = log softmax(W h_t)[y_t]`` come from the pinned
  cross-entropy oracle (``flce_oracle.forward`` in log-prob mode, with the same
  optional logit transform); tokens whose label is ``ignore_index`` are not
  completion tokens;
* the flattened batch is ``n_seq`` sequences of ``T / n_seq`` consecutive tokens;
  ``O_b`` are the completion tokens of sequence b and ``n_b = |O_b|``;
* GRPO (Shao et al. 2024, DeepSeekMath, the group relative policy optimisation
  objective with its unbiased KL estimator): with ratio
  ``r_t = exp(logp_t - old_t)`` (old = logp when not given, i.e. one update per
  batch), ``s_t = min(r_t A_b, clip(r_t, 1 - eps_low, 1 + eps_high) A_b)``,
  ``k_t = exp(ref_t - logp_t) - (ref_t - logp_t) - 1`` (0 without a reference),
  ``L = -(1 / B') sum_{b: n_b > 0} (1 / n_b) sum_{t in O_b} (s_t - beta k_t)``,
  B' the number of sequences with a completion token;
* DPO (Rafailov et al. 2023, the direct preference optimisation loss):
  ``2P`` sequences, the first P chosen and the last P rejected, pair i =
  (i, P + i); ``pi_b = sum_{t in O_b} logp_t``;
  ``Delta_i = beta ((pi_i - ref_i) - (pi_{P+i} - ref_{P+i}))`` and
  ``L = (1 / P) sum_i -log sigmoid(Delta_i)``;
* KTO (Ethayarajh et al. 2024, the Kahneman-Tversky optimisation loss):
  ``r_b = pi_b - ref_b``, reference point ``z0 = max(kl_ref, 0)`` (a detached
  estimate the caller supplies), ``v_b = lambda_D sigmoid(beta (r_b - z0))`` for
  desirable and ``lambda_U sigmoid(beta (z0 - r_b))`` for undesirable sequences,
  ``L = (1 / B) sum_b (lambda_b - v_b)``.

old, ref, the advantages and z0 are constants: gradients reach the policy's
hidden states and lm_head only, through ``dL/dlogp_t`` and the log-prob backward
(``flce_oracle.backward`` in log-prob mode with ``grad_out = dL/dlogp``).  At a
clipping kink (r A equal for both branches) the unclipped derivative is taken.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from oracle import flce_oracle as fo

IGNORE_INDEX = fo.IGNORE_INDEX


@dataclasses.dataclass
class PolicyLoss:
    loss: float
    dlogp: np.ndarray     # [T] dL/dlogp_t (0 off the completions)
    logp: np.ndarray      # [T] per-token log p of the label (0 off the completions)


def _sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0, 1.0 / (1.0 + np.exp(-np.abs(x))),
                    np.exp(-np.abs(x)) / (1.0 + np.exp(-np.abs(x))))


def _softplus(x):
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _layout(labels, n_seq: int, ignore_index: int):
    labels = np.asarray(labels, dtype=np.int64)
    T = labels.shape[0]
    if n_seq < 1 or T % n_seq:
        raise ValueError(f"T = {T} is not a multiple of n_seq = {n_seq}")
    S = T // n_seq
    mask = (labels != ignore_index).reshape(n_seq, S)
    return S, mask


def grpo_from_logp(logp, labels, n_seq: int, advantages, old_logp=None, ref_logp=None,
                   beta: float = 0.0, eps_low: float = 0.2, eps_high: float = 0.2,
                   ignore_index: int = IGNORE_INDEX) -> PolicyLoss:
    """GRPO loss and dL/dlogp from per-token log-probs (the objective written out)."""
    S, mask = _layout(labels, n_seq, ignore_index)
    lp = np.asarray(logp, dtype=np.float64).reshape(n_seq, S)
    old = lp if old_logp is None else np.asarray(old_logp, dtype=np.float64).reshape(n_seq, S)
    A = np.asarray(advantages, dtype=np.float64).reshape(n_seq, 1)
    r = np.exp(lp - old)
    unclipped = r * A
    clipped = np.clip(r, 1.0 - eps_low, 1.0 + eps_high) * A
    s = np.minimum(unclipped, clipped)
    ds = np.where(unclipped <= clipped, r * A, 0.0)
    if ref_logp is None:
        k = np.zeros_like(lp)
        dk = np.zeros_like(lp)
    else:
        d = np.asarray(ref_logp, dtype=np.float64).reshape(n_seq, S) - lp
        k = np.exp(d) - d - 1.0
        dk = 1.0 - np.exp(d)
    n = mask.sum(axis=1)
    used = n > 0
    n_used = int(used.sum())
    obj = np.where(mask, s - beta * k, 0.0)
    J = np.where(used, obj.sum(axis=1) / np.maximum(n, 1), 0.0)
    loss = float(-J[used].sum() / n_used) if n_used else 0.0
    scale = np.where(used, -1.0 / (max(n_used, 1) * np.maximum(n, 1)), 0.0)[:, None]
    dlogp = np.where(mask, scale * (ds - beta * dk), 0.0)
    return PolicyLoss(loss=loss, dlogp=dlogp.reshape(-1), logp=np.where(mask, lp, 0.0).reshape(-1))


def _seq_logp(logp, mask):
    return np.where(mask, logp, 0.0).sum(axis=1)


def dpo_from_logp(logp, labels, n_seq: int, ref_seq_logp, beta: float = 0.1,
                  ignore_index: int = IGNORE_INDEX) -> PolicyLoss:
    """DPO loss and dL/dlogp; sequences [0, P) are chosen, [P, 2P) rejected."""
    if n_seq % 2:
        raise ValueError("DPO needs an even number of sequences (chosen, then rejected)")
    S, mask = _layout(labels, n_seq, ignore_index)
    lp = np.asarray(logp, dtype=np.float64).reshape(n_seq, S)
    pi = _seq_logp(lp, mask)
    ref = np.asarray(ref_seq_logp, dtype=np.float64)
    P = n_seq // 2
    delta = beta * ((pi[:P] - ref[:P]) - (pi[P:] - ref[P:]))
    loss = float(_softplus(-delta).sum() / P)
    g = beta * _sigmoid(-delta) / P          # dL/dpi_rejected; dL/dpi_chosen = -g
    dpi = np.concatenate([-g, g])
    dlogp = np.where(mask, dpi[:, None], 0.0)
    return PolicyLoss(loss=loss, dlogp=dlogp.reshape(-1), logp=np.where(mask, lp, 0.0).reshape(-1))


def kto_from_logp(logp, labels, n_seq: int, ref_seq_logp, desirable, kl_ref: float = 0.0,
                  beta: float = 0.1, desirable_weight: float = 1.0,
                  undesirable_weight: float = 1.0, ignore_index: int = IGNORE_INDEX) -> PolicyLoss:
    """KTO loss and dL/dlogp with a caller-supplied reference point (clamped at 0)."""
    S, mask = _layout(labels, n_seq, ignore_index)
    lp = np.asarray(logp, dtype=np.float64).reshape(n_seq, S)
    r = _seq_logp(lp, mask) - np.asarray(ref_seq_logp, dtype=np.float64)
    z0 = max(float(kl_ref), 0.0)
    des = np.asarray(desirable).astype(bool)
    x = np.where(des, beta * (r - z0), beta * (z0 - r))
    lam = np.where(des, desirable_weight, undesirable_weight)
    sx = _sigmoid(x)
    loss = float((lam - lam * sx).sum() / n_seq)
    # d(-lam sigmoid(x))/dr = -lam sigmoid'(x) dx/dr, dx/dr = +beta (desirable) or -beta
    dr = -lam * sx * (1.0 - sx) * np.where(des, beta, -beta) / n_seq
    dlogp = np.where(mask, dr[:, None], 0.0)
    return PolicyLoss(loss=loss, dlogp=dlogp.reshape(-1), logp=np.where(mask, lp, 0.0).reshape(-1))


def logp(hidden, weight, labels, ignore_index: int = IGNORE_INDEX,
         transform: Optional[fo.LogitTransform] = None) -> np.ndarray:
    """Per-token log p(label) of the policy (0 off the completions), float64."""
    return fo.forward(hidden, weight, labels, ignore_index, "logprob", transform).out


def grads(hidden, weight, labels, dlogp, grad_loss: float = 1.0,
          ignore_index: int = IGNORE_INDEX, transform: Optional[fo.LogitTransform] = None):
    """(dH, dW) of grad_loss * L given dL/dlogp: the log-prob backward of the LM head."""
    g = np.asarray(dlogp, dtype=np.float64) * float(grad_loss)
    return fo.backward(hidden, weight, labels, ignore_index, "logprob", grad_out=g,
                       transform=transform)
