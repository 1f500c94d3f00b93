"""Seeded synthetic inputs for the chunked LM-head + cross-entropy path.

This module only draws inputs: hidden states, lm_head weights, labels, the
ignore set and per-token upstream gradients.  It holds none of the loss
arithmetic, so both the CPU oracle and the HIP path can consume exactly the
same bits without sharing any of the computation under test.

Workload shapes follow the pages:

* the TRL single-chunk micro-benchmark, 256 tokens x 248,320 vocab x 2,048
  hidden (TRL v1.13 article, section on the chunked loss returning to tensor
  cores);
* a 16,384-token SFT step at Qwen3-8B's lm_head shape (same section, the
  end-to-end tokens/s table) with 256-row chunks (same article, section on the
  four hurdles, the ``chunked_nll`` paragraph);
* the GRPO selective log-prob example of batch 4 x context 8,192 x vocab
  128,000 (Unsloth GRPO long-context page, section on flattened sequence
  chunking, Equation 1 example);
* a 131,072-token single sequence (TRL v1.13 article, context-parallel step
  times at 131k tokens).

The pages print no value distributions; the ones used here are fixed by the
workload table of this repository's design notes: hidden ~ N(0, 1), lm_head
~ N(0, sigma^2), labels uniform over the vocabulary, an exact number of
ignored tokens chosen by a seeded permutation.

Random streams.  Every tensor gets its own child of one ``SeedSequence`` so
that changing one shape never changes another tensor's values, and large
matrices are drawn in fixed row blocks, each from its own grandchild stream, so
they can be filled by several threads with a result that does not depend on
the thread count.  Floats are drawn in float32 and rounded to bfloat16 with
round-to-nearest-even on the bit pattern (what ``Tensor.to(torch.bfloat16)``
does); they are returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Optional

import numpy as np

IGNORE_INDEX = -100
BLOCK_ROWS = 2048  # rows per independent random stream in a matrix


@dataclasses.dataclass(frozen=True)
class Workload:
    """A synthetic workload: shapes, value distribution and loss mode."""

    name: str
    T: int                 # flattened tokens (batch x sequence)
    H: int                 # hidden size
    V: int                 # vocabulary size
    chunk_rows: int        # rows per logit chunk (bounds live logit memory)
    w_std: float           # lm_head entries ~ N(0, w_std^2)
    ignore_count: int      # tokens whose label is IGNORE_INDEX
    mode: str              # "nll" or "logprob"
    reduction: str         # "mean" (scalar loss) or "none" (per-token upstream grad)
    seed: int
    seq_len: int = 0       # tokens per sequence, when the grad has prompt zeros
    prompt_len: int = 0    # leading tokens per sequence whose upstream grad is 0


def _ignored(T: int, frac: float) -> int:
    return int(round(frac * T))


WORKLOADS = {
    "tiny": Workload("tiny", T=67, H=128, V=1000, chunk_rows=16,
                     w_std=1.0 / math.sqrt(128), ignore_count=_ignored(67, 0.10),
                     mode="nll", reduction="mean", seed=1001),
    "single_chunk": Workload("single_chunk", T=256, H=2048, V=248320, chunk_rows=256,
                             w_std=0.02, ignore_count=0, mode="nll", reduction="mean",
                             seed=1002),
    "qwen3_8b_sft": Workload("qwen3_8b_sft", T=16384, H=4096, V=151936, chunk_rows=256,
                             w_std=0.02, ignore_count=_ignored(16384, 0.05),
                             mode="nll", reduction="mean", seed=1003),
    "grpo_logprob": Workload("grpo_logprob", T=32768, H=4096, V=128000, chunk_rows=256,
                             w_std=0.02, ignore_count=0, mode="logprob", reduction="none",
                             seed=1004, seq_len=8192, prompt_len=1024),
    "long_context": Workload("long_context", T=131072, H=4096, V=151936, chunk_rows=256,
                             w_std=0.02, ignore_count=0, mode="nll", reduction="mean",
                             seed=1005),
}


def custom(name: str, T: int, H: int, V: int, *, chunk_rows: int = 256,
           w_std: Optional[float] = None, ignore_frac: float = 0.0,
           mode: str = "nll", reduction: str = "mean", seed: int = 7,
           seq_len: int = 0, prompt_len: int = 0) -> Workload:
    """A workload of arbitrary shape with the same recipe (for tests)."""
    if w_std is None:
        w_std = 1.0 / math.sqrt(H)
    return Workload(name, T=T, H=H, V=V, chunk_rows=chunk_rows, w_std=w_std,
                    ignore_count=_ignored(T, ignore_frac), mode=mode,
                    reduction=reduction, seed=seed, seq_len=seq_len,
                    prompt_len=prompt_len)


@dataclasses.dataclass
class Inputs:
    workload: Workload
    hidden: np.ndarray            # uint16 bf16 bits [T, H]
    weight: np.ndarray            # uint16 bf16 bits [V, H]
    labels: np.ndarray            # int64 [T], IGNORE_INDEX where ignored
    grad_out: Optional[np.ndarray]  # float32 [T] upstream dL/d out, or None (mean)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16_matrix(seq: np.random.SeedSequence, rows: int, cols: int,
                       std: float) -> np.ndarray:
    """rows x cols bf16 bits of std * N(0, 1) drawn in float32, block-seeded."""
    out = np.empty((rows, cols), dtype=np.uint16)
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    children = seq.spawn(nblk) if nblk else []
    scale = np.float32(std)

    def fill(b: int) -> None:
        r0 = b * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        g = np.random.default_rng(children[b])
        x = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            x *= scale
        out[r0:r1] = round_to_bf16_bits(x)

    if nblk <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def make_inputs(w: Workload, *, zero_weight: bool = False) -> Inputs:
    """Draw the inputs of workload ``w``.

    ``zero_weight`` replaces the lm_head by zeros (all other draws unchanged),
    a degenerate case with a closed-form answer.
    """
    root = np.random.SeedSequence(w.seed)
    s_hidden, s_weight, s_labels, s_ignore, s_grad = root.spawn(5)
    hidden = normal_bf16_matrix(s_hidden, w.T, w.H, 1.0)
    if zero_weight:
        weight = np.zeros((w.V, w.H), dtype=np.uint16)
    else:
        weight = normal_bf16_matrix(s_weight, w.V, w.H, w.w_std)
    labels = np.random.default_rng(s_labels).integers(0, w.V, size=w.T, dtype=np.int64)
    if w.ignore_count:
        idx = np.random.default_rng(s_ignore).permutation(w.T)[: w.ignore_count]
        labels[idx] = IGNORE_INDEX
    grad = None
    if w.reduction == "none":
        grad = np.random.default_rng(s_grad).standard_normal(w.T, dtype=np.float32)
        if w.seq_len and w.prompt_len:
            pos = np.arange(w.T) % w.seq_len
            grad[pos < w.prompt_len] = 0.0
    return Inputs(w, hidden, weight, labels, grad)


# ---------------------------------------------------------------------------
# Distillation: a student head and a teacher head over the same vocabulary.
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class DistillWorkload:
    """Student and teacher hidden states / lm_heads over one vocabulary."""

    name: str
    T: int                 # flattened tokens
    Hs: int                # student hidden size
    Ht: int                # teacher hidden size
    V: int                 # shared vocabulary
    chunk_rows: int        # rows per logit chunk (bounds live logit memory)
    ws_std: float          # student lm_head entries ~ N(0, ws_std^2)
    wt_std: float          # teacher lm_head entries ~ N(0, wt_std^2)
    ignore_count: int      # tokens left out of the loss (mask = IGNORE_INDEX)
    seed: int
    reduction: str = "mean"  # "mean" (scalar loss) or "none" (per-token upstream grad)


DISTILL_WORKLOADS = {
    "distill_tiny": DistillWorkload("distill_tiny", T=67, Hs=128, Ht=192, V=1000, chunk_rows=16,
                                    ws_std=1.0 / math.sqrt(128), wt_std=1.0 / math.sqrt(192),
                                    ignore_count=_ignored(67, 0.10), seed=2001),
    # student at the Qwen3-8B lm_head shape, a wider teacher over the same vocabulary
    "distill_qwen3": DistillWorkload("distill_qwen3", T=16384, Hs=4096, Ht=5120, V=151936,
                                     chunk_rows=256, ws_std=0.02, wt_std=0.02,
                                     ignore_count=_ignored(16384, 0.05), seed=2002),
}


def distill_custom(name: str, T: int, Hs: int, Ht: int, V: int, *, chunk_rows: int = 256,
                   ws_std: Optional[float] = None, wt_std: Optional[float] = None,
                   ignore_frac: float = 0.0, reduction: str = "mean",
                   seed: int = 7) -> DistillWorkload:
    """A distillation workload of arbitrary shape with the same recipe (for tests)."""
    return DistillWorkload(name, T=T, Hs=Hs, Ht=Ht, V=V, chunk_rows=chunk_rows,
                           ws_std=1.0 / math.sqrt(Hs) if ws_std is None else ws_std,
                           wt_std=1.0 / math.sqrt(Ht) if wt_std is None else wt_std,
                           ignore_count=_ignored(T, ignore_frac), seed=seed,
                           reduction=reduction)


@dataclasses.dataclass
class DistillInputs:
    workload: DistillWorkload
    s_hidden: np.ndarray          # uint16 bf16 bits [T, Hs]
    s_weight: np.ndarray          # uint16 bf16 bits [V, Hs]
    t_hidden: np.ndarray          # uint16 bf16 bits [T, Ht]
    t_weight: np.ndarray          # uint16 bf16 bits [V, Ht]
    labels: np.ndarray            # int64 [T]: IGNORE_INDEX for left-out tokens, else 0
    grad_out: Optional[np.ndarray]  # float32 [T] upstream dL/d kl, or None (mean)


def make_distill_inputs(w: DistillWorkload) -> DistillInputs:
    """Draw the inputs of distillation workload ``w`` (hidden ~ N(0, 1))."""
    root = np.random.SeedSequence(w.seed)
    s_sh, s_sw, s_th, s_tw, s_ign, s_grad = root.spawn(6)
    s_hidden = normal_bf16_matrix(s_sh, w.T, w.Hs, 1.0)
    s_weight = normal_bf16_matrix(s_sw, w.V, w.Hs, w.ws_std)
    t_hidden = normal_bf16_matrix(s_th, w.T, w.Ht, 1.0)
    t_weight = normal_bf16_matrix(s_tw, w.V, w.Ht, w.wt_std)
    labels = np.zeros(w.T, dtype=np.int64)
    if w.ignore_count:
        idx = np.random.default_rng(s_ign).permutation(w.T)[: w.ignore_count]
        labels[idx] = IGNORE_INDEX
    grad = None
    if w.reduction == "none":
        grad = np.random.default_rng(s_grad).standard_normal(w.T, dtype=np.float32)
    return DistillInputs(w, s_hidden, s_weight, t_hidden, t_weight, labels, grad)


# ---------------------------------------------------------------------------
# Policy-optimisation losses: the flattened batch is n_seq sequences of
# seq_len tokens whose first prompt_len tokens are the prompt (label =
# IGNORE_INDEX, not completion tokens); per-sequence and per-token side inputs
# are standard normals that a caller scales and offsets (e.g. old log-probs =
# the policy's log-probs + sigma * old_noise).
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class PolicyWorkload:
    name: str
    n_seq: int
    seq_len: int
    prompt_len: int
    H: int
    V: int
    chunk_rows: int
    w_std: float
    seed: int

    @property
    def T(self) -> int:
        return self.n_seq * self.seq_len


POLICY_WORKLOADS = {
    # the GRPO log-prob example (batch 4 x context 8,192 x vocab 128,000, hidden 4,096)
    "grpo_qwen3": PolicyWorkload("grpo_qwen3", n_seq=4, seq_len=8192, prompt_len=1024, H=4096,
                                 V=128000, chunk_rows=256, w_std=0.02, seed=3001),
}


def policy_custom(name: str, n_seq: int, seq_len: int, prompt_len: int, H: int, V: int, *,
                  chunk_rows: int = 256, w_std: Optional[float] = None,
                  seed: int = 7) -> PolicyWorkload:
    return PolicyWorkload(name, n_seq=n_seq, seq_len=seq_len, prompt_len=prompt_len, H=H, V=V,
                          chunk_rows=chunk_rows,
                          w_std=1.0 / math.sqrt(H) if w_std is None else w_std, seed=seed)


@dataclasses.dataclass
class PolicyInputs:
    workload: PolicyWorkload
    hidden: np.ndarray        # uint16 bf16 bits [T, H]
    weight: np.ndarray        # uint16 bf16 bits [V, H]
    labels: np.ndarray        # int64 [T]: completion ids, IGNORE_INDEX on the prompts
    advantages: np.ndarray    # float32 [n_seq] ~ N(0, 1)
    old_noise: np.ndarray     # float32 [T] ~ N(0, 1)
    ref_noise: np.ndarray     # float32 [T] ~ N(0, 1)
    seq_noise: np.ndarray     # float32 [n_seq] ~ N(0, 1)
    desirable: np.ndarray     # uint8 [n_seq], each 1 with probability 1/2


def make_policy_inputs(w: PolicyWorkload) -> PolicyInputs:
    root = np.random.SeedSequence(w.seed)
    s_h, s_w, s_y, s_a, s_o, s_r, s_s, s_d = root.spawn(8)
    hidden = normal_bf16_matrix(s_h, w.T, w.H, 1.0)
    weight = normal_bf16_matrix(s_w, w.V, w.H, w.w_std)
    labels = np.random.default_rng(s_y).integers(0, w.V, size=w.T, dtype=np.int64)
    labels[(np.arange(w.T) % w.seq_len) < w.prompt_len] = IGNORE_INDEX
    f32 = np.float32
    return PolicyInputs(
        w, hidden, weight, labels,
        advantages=np.random.default_rng(s_a).standard_normal(w.n_seq, dtype=f32),
        old_noise=np.random.default_rng(s_o).standard_normal(w.T, dtype=f32),
        ref_noise=np.random.default_rng(s_r).standard_normal(w.T, dtype=f32),
        seq_noise=np.random.default_rng(s_s).standard_normal(w.n_seq, dtype=f32),
        desirable=(np.random.default_rng(s_d).random(w.n_seq) < 0.5).astype(np.uint8))
