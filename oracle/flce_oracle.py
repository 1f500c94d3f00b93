"""CPU oracle for chunked fused linear cross-entropy / selective log-softmax.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module; the product path never does.
It shares no code with the HIP library and imports nothing from it.

What it computes (a plain, slow, obviously correct definition in float64):

* Unsloth's GRPO long-context page, section "Chunking der abgeflachten
  Sequenzlaenge": the chunked call multiplies each chunk of the flattened
  hidden states by the lm_head, upcasts the chunk logits to float32 and returns
  the selective log-softmax at the completion ids.  Chunking over rows only
  changes the schedule (the page says it adds no peak memory and loses no
  accuracy), so the oracle takes the whole row of logits at once:
  ``z = h @ W^T``, ``lse = max z + ln sum exp(z - max z)``, ``log p(y) = z_y - lse``.
* TRL v1.13 article, section on the four hurdles: ``loss_type="chunked_nll"``
  computes the NLL of 256 rows at a time and sums; NLL is ``lse - z_y``.
* Unsloth page, section "Auslagern von Aktivierungen fuer Log-Softmax": the
  backward recomputes the chunked call and back-propagates the per-token
  ``grad_output``.  With ``P = softmax(z)`` the gradient of NLL with respect to
  ``z`` is ``P - onehot(y)`` and that of ``log p(y)`` is ``onehot(y) - P``, so
  ``G = c_t (P - onehot)`` with ``c_t = g_t`` (NLL) or ``-g_t`` (log-prob), and
  ``dH = G W``, ``dW = G^T H``.
* TRL v1.13 article, section on the chunked loss returning to tensor cores:
  the operands stay bf16 and are never upcast to float32 GEMM operands; the
  oracle decodes the same bf16 bits exactly into float64 (bf16 -> fp32 is a
  16-bit shift and fp32 is a subset of fp64), so it sees the GPU's inputs.

* Same Unsloth section, the compiled chunked call and the list under it: the
  call takes ``logit_scale_multiply``, ``logit_scale_divide``,
  ``logit_softcapping`` and ``temperature``, and the page says softcapping and
  temperature scaling are supported.  The page gives the names only; the
  oracle applies them to each logit in that order (see ``LogitTransform``)
  before the log-softmax, and the backward takes the chain rule through them.

Readings where the pages are silent (each one is listed with its reason in the
design notes):

* ``ignore_index`` tokens output 0, get a zero gradient row and are left out
  of the mean's denominator (PyTorch's convention; the pages never mention it).
* the mean divides by the number of non-ignored tokens; with none, the mean is
  0 and the gradients are 0 (PyTorch would give NaN).
* a label outside ``[0, V)`` that is not ``ignore_index`` is a caller error:
  the oracle raises.
* logit transforms: ``z' = z * multiply`` (if multiply != 0), ``/ divide`` (if
  divide != 0), ``cap * tanh(z' / cap)`` (if cap != 0), ``/ temperature``, in
  that order; 0 means "not applied" for the first three, temperature must be
  positive and the others non-negative.

Large inputs are processed in row blocks of complete vocabulary rows so that
memory stays bounded; a block is a schedule detail, not part of the method.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

IGNORE_INDEX = -100
_BLOCK_ELEMS = 1 << 27  # float64 logits per row block (1 GiB)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("expected uint16 bf16 bit patterns")
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def _as_f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return x.astype(np.float64, copy=False)


def _rows_per_block(V: int, T: int) -> int:
    return max(1, min(T, _BLOCK_ELEMS // max(1, V)))


def valid_mask(labels: np.ndarray, V: int, ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """True where the label is used; raises on an out-of-range used label."""
    labels = np.asarray(labels, dtype=np.int64)
    valid = labels != ignore_index
    bad = valid & ((labels < 0) | (labels >= V))
    if bad.any():
        raise ValueError(f"label out of range [0, {V}) at tokens {np.nonzero(bad)[0][:8]}")
    return valid


@dataclasses.dataclass(frozen=True)
class LogitTransform:
    """Per-logit transform of the chunked call's keyword arguments (0: not applied)."""
    scale_multiply: float = 0.0
    scale_divide: float = 0.0
    softcap: float = 0.0
    temperature: float = 1.0

    def check(self) -> None:
        if not self.temperature > 0.0:
            raise ValueError("temperature must be positive")
        for name in ("scale_multiply", "scale_divide", "softcap"):
            if not getattr(self, name) >= 0.0:
                raise ValueError(f"{name} must be non-negative")

    def apply(self, z: np.ndarray):
        """(z', dz'/dz) elementwise, float64."""
        self.check()
        x = np.asarray(z, dtype=np.float64)
        d = np.ones_like(x)
        if self.scale_multiply != 0.0:
            x = x * self.scale_multiply
            d = d * self.scale_multiply
        if self.scale_divide != 0.0:
            x = x / self.scale_divide
            d = d / self.scale_divide
        if self.softcap != 0.0:
            t = np.tanh(x / self.softcap)
            x = self.softcap * t
            d = d * (1.0 - t * t)
        if self.temperature != 1.0:
            x = x / self.temperature
            d = d / self.temperature
        return x, d


def _logits(h: np.ndarray, w: np.ndarray, transform: Optional[LogitTransform]):
    """Transformed logit rows and their derivative (None when untransformed)."""
    z = h @ w.T
    if transform is None:
        return z, None
    return transform.apply(z)


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """Textbook max-shifted log-sum-exp over the last axis (float64)."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


@dataclasses.dataclass
class Forward:
    out: np.ndarray    # [T] per-token NLL or log-prob, 0 where ignored
    lse: np.ndarray    # [T] log-sum-exp of the logit row (also for ignored rows)
    mean: float        # sum of out over used tokens / number of used tokens (0 if none)
    n_valid: int


def forward(hidden, weight, labels, ignore_index: int = IGNORE_INDEX,
            mode: str = "nll", transform: Optional[LogitTransform] = None) -> Forward:
    """Per-token NLL (``mode="nll"``) or log p(label) (``mode="logprob"``) of the
    (optionally transformed) logits."""
    if mode not in ("nll", "logprob"):
        raise ValueError(mode)
    h = _as_f64(hidden)
    w = _as_f64(weight)
    labels = np.asarray(labels, dtype=np.int64)
    T, V = h.shape[0], w.shape[0]
    valid = valid_mask(labels, V, ignore_index)
    lse = np.empty(T)
    zy = np.zeros(T)
    step = _rows_per_block(V, T)
    for r0 in range(0, T, step):
        r1 = min(T, r0 + step)
        z, _ = _logits(h[r0:r1], w, transform)  # full-vocabulary logit rows
        lse[r0:r1] = logsumexp_rows(z)
        rows = np.nonzero(valid[r0:r1])[0]
        zy[r0 + rows] = z[rows, labels[r0 + rows]]
    nll = lse - zy
    out = np.where(valid, nll if mode == "nll" else -nll, 0.0)
    n_valid = int(valid.sum())
    mean = float(out[valid].sum() / n_valid) if n_valid else 0.0
    return Forward(out=out, lse=lse, mean=mean, n_valid=n_valid)


def token_scale(labels, V: int, ignore_index: int = IGNORE_INDEX, mode: str = "nll",
                grad_out: Optional[np.ndarray] = None,
                grad_mean: Optional[float] = None) -> np.ndarray:
    """c_t with G_t = c_t (P_t - onehot(y_t)).

    ``grad_out`` is dL/d out_t per token; if it is None, ``grad_mean`` (default
    1) is dL/d mean and each used token gets grad_mean / n_valid.
    """
    valid = valid_mask(labels, V, ignore_index)
    if grad_out is not None:
        g = np.asarray(grad_out, dtype=np.float64).copy()
    else:
        n_valid = int(valid.sum())
        gm = 1.0 if grad_mean is None else float(grad_mean)
        g = np.full(valid.shape, gm / n_valid if n_valid else 0.0)
    if mode == "logprob":
        g = -g
    return np.where(valid, g, 0.0)


def grad_logits(z: np.ndarray, lse: np.ndarray, labels: np.ndarray, c: np.ndarray,
                dz: Optional[np.ndarray] = None) -> np.ndarray:
    """G = c_t (softmax(z_t) - onehot(y_t)) for a block of rows; with a logit
    transform, z are the transformed logits and the chain rule multiplies by
    dz = dz'/dz (the gradient with respect to the raw logits)."""
    g = np.exp(z - lse[:, None])
    rows = np.nonzero(c != 0.0)[0]
    g[rows, labels[rows]] -= 1.0
    g = g * c[:, None]
    return g if dz is None else g * dz


def backward(hidden, weight, labels, ignore_index: int = IGNORE_INDEX, mode: str = "nll",
             grad_out: Optional[np.ndarray] = None, grad_mean: Optional[float] = None,
             lse: Optional[np.ndarray] = None, transform: Optional[LogitTransform] = None):
    """(dH [T, H], dW [V, H]) in float64 for the loss the forward defines."""
    h = _as_f64(hidden)
    w = _as_f64(weight)
    labels = np.asarray(labels, dtype=np.int64)
    T, V = h.shape[0], w.shape[0]
    c = token_scale(labels, V, ignore_index, mode, grad_out, grad_mean)
    dh = np.zeros_like(h)
    dw = np.zeros_like(w)
    step = _rows_per_block(V, T)
    for r0 in range(0, T, step):
        r1 = min(T, r0 + step)
        z, dz = _logits(h[r0:r1], w, transform)
        l = logsumexp_rows(z) if lse is None else np.asarray(lse[r0:r1], dtype=np.float64)
        g = grad_logits(z, l, labels[r0:r1], c[r0:r1], dz)
        dh[r0:r1] = g @ w
        dw += g.T @ h[r0:r1]
    return dh, dw


def forward_rows(hidden, weight, labels, rows: Sequence[int], ignore_index: int = IGNORE_INDEX,
                 mode: str = "nll", transform: Optional[LogitTransform] = None):
    """(out, lse) of the selected tokens only; each row needs its own logits only."""
    rows = np.asarray(rows, dtype=np.int64)
    f = forward(np.asarray(hidden)[rows], weight, np.asarray(labels)[rows], ignore_index, mode,
                transform)
    return f.out, f.lse


def grad_hidden_rows(hidden, weight, labels, rows: Sequence[int], c_rows: np.ndarray,
                     ignore_index: int = IGNORE_INDEX,
                     transform: Optional[LogitTransform] = None) -> np.ndarray:
    """dH rows of the selected tokens given their scales c_t (a row needs only its logits)."""
    rows = np.asarray(rows, dtype=np.int64)
    h = _as_f64(np.asarray(hidden)[rows])
    w = _as_f64(weight)
    lab = np.asarray(labels, dtype=np.int64)[rows]
    valid_mask(lab, w.shape[0], ignore_index)
    z, dz = _logits(h, w, transform)
    g = grad_logits(z, logsumexp_rows(z), lab, np.asarray(c_rows, dtype=np.float64), dz)
    return g @ w


def grad_weight_rows(hidden, weight, labels, vocab_rows: Sequence[int], c: np.ndarray,
                     lse: np.ndarray, transform: Optional[LogitTransform] = None) -> np.ndarray:
    """dW rows of the selected vocabulary entries: dW_v = sum_t G_tv H_t.

    Needs lse for every token (from ``forward``); only the selected columns of
    the logits are formed.
    """
    vr = np.asarray(vocab_rows, dtype=np.int64)
    h = _as_f64(hidden)
    wv = _as_f64(np.asarray(weight)[vr])
    labels = np.asarray(labels, dtype=np.int64)
    c = np.asarray(c, dtype=np.float64)
    z, dz = _logits(h, wv, transform)              # [T, len(vr)]
    g = np.exp(z - np.asarray(lse, dtype=np.float64)[:, None])
    g -= (labels[:, None] == vr[None, :])
    g *= c[:, None]
    if dz is not None:
        g *= dz
    return g.T @ h


# --- logit-memory formulas (Unsloth page, section "Chunking der abgeflachten
# Sequenzlaenge", Equations 1-3, and section "Chunking der Hidden States") ---

GIB = 1024.0 ** 3


def logit_memory_eq1(batch: int, context: int, vocab: int, bytes_per_elem: float = 1.0) -> float:
    """Equation 1: all logits of the batch, in GiB (the page's formula has no byte factor)."""
    return batch * context * vocab * bytes_per_elem / GIB


def logit_memory_eq2(context: int, vocab: int, bytes_per_elem: float = 1.0) -> float:
    """Equation 2: one batch sample at a time."""
    return context * vocab * bytes_per_elem / GIB


def logit_memory_eq3(context: int, vocab: int, multiplier: int, bytes_per_elem: float = 1.0) -> float:
    """Equation 3: one sample split into ``multiplier`` sequence chunks."""
    return (context / multiplier) * vocab * bytes_per_elem / GIB


def hidden_memory(batch: int, context: int, hidden_dim: int, bytes_per_elem: float = 1.0) -> float:
    """Hidden-state memory formula of the same page, in GiB."""
    return batch * context * hidden_dim * bytes_per_elem / GIB


def default_multiplier(context: int) -> int:
    """The page's default chunk multiplier, max(4, context // 4096)."""
    return max(4, context // 4096)
