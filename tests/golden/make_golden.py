"""Write oracle values for the full-size workloads (run on the CPU; calls only the oracle).

For each workload the inputs are re-drawn with the seeded generator and the
float64 oracle computes, over ALL tokens and the FULL vocabulary:
  * the per-token output and lse of a sample of tokens, and the mean;
  * the grad_hidden rows of those tokens;
  * the grad_weight rows of a sample of vocabulary entries (these need the
    lse of every token, hence the full forward).
The samples include the first and last tokens and vocabulary rows, tile
boundaries, the ragged tail, ignored tokens and labels of sampled tokens, and the
tokens on both sides of every multiple of 8,192 (the backward's row blocks).  The
vocabulary rows on both sides of every multiple of 4,096 (and of 7,936 where
V = 128,000) cover the backward's vocabulary chunks, all multiples of 256 rows: their
dW rows are kept for the first 512 hidden columns (``vocab_edge``, ``dw_edge``).

Variants with a logit transform (the chunked call's multiply / divide /
softcap / temperature keywords on the Unsloth GRPO page) reuse a workload's
inputs; the transform's values are stored in the file beside the results.  The
softcap variant caps at about four standard deviations of these logits, so the
tanh is far from linear over the top of each row.

Usage:  python tests/golden/make_golden.py [workload ...]
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from chunked_lm_head_amd import synth  # noqa: E402  (inputs only)
from oracle import distill_oracle as dst  # noqa: E402
from oracle import flce_oracle as o  # noqa: E402
from oracle import policy_oracle as po  # noqa: E402

FULL = ("single_chunk", "qwen3_8b_sft", "grpo_logprob", "long_context")
# name -> (workload, transform)
VARIANTS = {
    "qwen3_8b_sft_softcap": ("qwen3_8b_sft", dict(softcap=5.0, temperature=0.7)),
    "single_chunk_scaled": ("single_chunk",
                            dict(scale_multiply=1.5, scale_divide=1.2, temperature=0.8)),
}


def sample_tokens(w: synth.Workload, labels: np.ndarray, rng) -> np.ndarray:
    T = w.T
    picks = {0, 1, 255, 256, T // 2, T - 1, T - 2}
    picks |= {T - 1 - int(i) for i in range(0, min(T, 300), 37)}     # ragged / last tile
    for k in range(8192, T, 8192):                                    # row-block edges
        picks |= {k - 1, k}
    ign = np.nonzero(labels == synth.IGNORE_INDEX)[0]
    picks |= set(int(i) for i in ign[:3])
    if getattr(w, "prompt_len", 0):
        picks |= {w.seq_len + 5, w.prompt_len - 1, w.prompt_len}    # zero / nonzero grads
    while len(picks) < 24:
        picks.add(int(rng.integers(0, T)))
    return np.array(sorted(p for p in picks if 0 <= p < T), dtype=np.int64)


def sample_vocab(w: synth.Workload, labels: np.ndarray, tokens: np.ndarray, rng) -> np.ndarray:
    V = w.V
    picks = {0, 255, 256, V - 1, V - 2}
    used = labels[tokens][labels[tokens] != synth.IGNORE_INDEX]
    picks |= set(int(x) for x in used[:4])
    while len(picks) < 12:
        picks.add(int(rng.integers(0, V)))
    return np.array(sorted(picks), dtype=np.int64)


EDGE_COLS = 512


def vocab_edges(V: int) -> np.ndarray:
    """Vocabulary rows on both sides of each multiple of 4,096, and of 7,936 when
    V = 128,000: the edges of every vocabulary chunk the backward can use here."""
    steps = (4096, 7936) if V == 128000 else (4096,)
    picks = set()
    for m in steps:
        for k in range(m, V, m):
            picks |= {k - 1, k}
    return np.array(sorted(picks), dtype=np.int64)


def make(name: str) -> str:
    base, xf = VARIANTS.get(name, (name, {}))
    w = synth.WORKLOADS[base]
    tr = o.LogitTransform(**xf) if xf else None
    t0 = time.time()
    x = synth.make_inputs(w)
    rng = np.random.default_rng(w.seed + 77)
    f = o.forward(x.hidden, x.weight, x.labels, synth.IGNORE_INDEX, w.mode, transform=tr)
    tokens = sample_tokens(w, x.labels, rng)
    vocab = sample_vocab(w, x.labels, tokens, rng)
    if w.reduction == "mean":
        c = o.token_scale(x.labels, w.V, synth.IGNORE_INDEX, w.mode, grad_mean=1.0)
    else:
        c = o.token_scale(x.labels, w.V, synth.IGNORE_INDEX, w.mode, grad_out=x.grad_out)
    dh = o.grad_hidden_rows(x.hidden, x.weight, x.labels, tokens, c[tokens], synth.IGNORE_INDEX,
                            transform=tr)
    dw = o.grad_weight_rows(x.hidden, x.weight, x.labels, vocab, c, f.lse, transform=tr)
    edges = vocab_edges(w.V)
    dw_edge = o.grad_weight_rows(x.hidden, x.weight, x.labels, edges, c, f.lse,
                                 transform=tr)[:, :EDGE_COLS]
    tv = o.LogitTransform(**xf)
    path = os.path.join(HERE, f"{name}.npz")
    np.savez(path, tokens=tokens, out=f.out[tokens], lse=f.lse[tokens], mean=np.float64(f.mean),
             n_valid=np.int64(f.n_valid), vocab=vocab, dh=dh.astype(np.float32),
             dw=dw.astype(np.float32), dw_norm_rows=np.linalg.norm(dw, axis=1),
             vocab_edge=edges, dw_edge=dw_edge.astype(np.float32),
             seed=np.int64(w.seed), workload=np.str_(base),
             transform=np.array([tv.scale_multiply, tv.scale_divide, tv.softcap,
                                 tv.temperature], dtype=np.float64))
    print(f"{name}: {time.time() - t0:.0f} s -> {path}", flush=True)
    return path


DISTILL = ("distill_qwen3", "distill_qwen3_jsd")
# name -> (workload, divergence, beta)
DISTILL_VARIANTS = {"distill_qwen3": ("distill_qwen3", "kl", 0.5),
                    "distill_qwen3_jsd": ("distill_qwen3", "jsd", 0.5)}


def make_distill(name: str) -> str:
    """Distillation workload: sampled per-token divergence (KL, or the JSD with its
    weight beta) and log-sum-exps, the mean, the student's dH rows of the sampled
    tokens and dW rows of sampled vocabulary entries (those need both log-sum-exps
    of every token, and for the JSD each token's gbar)."""
    base, divergence, beta = DISTILL_VARIANTS[name]
    kw = dict(divergence=divergence, beta=beta)
    w = synth.DISTILL_WORKLOADS[base]
    t0 = time.time()
    x = synth.make_distill_inputs(w)
    rng = np.random.default_rng(w.seed + 77)
    f = dst.forward(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, x.labels, **kw)
    tokens = sample_tokens(w, x.labels, rng)
    picks = {0, 255, 256, w.V - 1, w.V - 2}
    while len(picks) < 12:
        picks.add(int(rng.integers(0, w.V)))
    vocab = np.array(sorted(picks), dtype=np.int64)
    c = dst.token_scale(x.labels, w.T, grad_mean=1.0)
    dh = dst.grad_hidden_rows(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, tokens, c[tokens],
                              **kw)
    gbar = (dst.jsd_gbar(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, beta=beta)
            if divergence == "jsd" else None)
    dw = dst.grad_weight_rows(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, vocab, c,
                              f.lse_s, f.lse_t, gbar=gbar, **kw)
    edges = vocab_edges(w.V)
    dw_edge = dst.grad_weight_rows(x.s_hidden, x.s_weight, x.t_hidden, x.t_weight, edges, c,
                                   f.lse_s, f.lse_t, gbar=gbar, **kw)[:, :EDGE_COLS]
    path = os.path.join(HERE, f"{name}.npz")
    np.savez(path, tokens=tokens, kl=f.kl[tokens], lse_s=f.lse_s[tokens], lse_t=f.lse_t[tokens],
             mean=np.float64(f.mean), n_valid=np.int64(f.n_valid), vocab=vocab,
             dh=dh.astype(np.float32), dw=dw.astype(np.float32), seed=np.int64(w.seed),
             workload=np.str_(base), divergence=np.str_(divergence), beta=np.float64(beta),
             vocab_edge=edges, dw_edge=dw_edge.astype(np.float32))
    print(f"{name}: {time.time() - t0:.0f} s -> {path}", flush=True)
    return path


POLICY = ("grpo_qwen3",)
# loss parameters of the policy goldens (GRPO: DeepSeekMath's beta and clip range)
POLICY_PARAMS = dict(grpo_beta=0.04, eps_low=0.2, eps_high=0.2, dpo_beta=0.1, kto_beta=0.1,
                     kl_ref=0.05, desirable_weight=1.0, undesirable_weight=1.33)
GRAD_LOSS = 1.0


def kink_free_old(lp, old, eps_low, eps_high, mask):
    """Shift float32 old log-probs until no ratio lies within 1e-3 of a clip bound, so that
    fp32 and fp64 log-probs take the same branch of the clipped surrogate."""
    old = old.copy()
    for _ in range(10):
        r = np.exp(lp - old.astype(np.float64))
        near = ((np.abs(r - (1 + eps_high)) < 1e-3) | (np.abs(r - (1 - eps_low)) < 1e-3)) & mask
        if not near.any():
            return old
        old[near] += np.float32(0.01)
    raise RuntimeError("could not move the ratios off the clipping bounds")


def make_policy(name: str) -> str:
    """GRPO, DPO and KTO at full size from one float64 forward over all tokens: the
    side inputs built from the oracle's log-probs (old and reference log-probs, reference
    sequence log-probs), each loss, and for each the dH rows of sampled tokens and the dW
    rows of sampled vocabulary entries (those need every token's lse and dL/dlogp)."""
    w = synth.POLICY_WORKLOADS[name]
    P = POLICY_PARAMS
    t0 = time.time()
    x = synth.make_policy_inputs(w)
    rng = np.random.default_rng(w.seed + 77)
    f = o.forward(x.hidden, x.weight, x.labels, synth.IGNORE_INDEX, "logprob")
    lp = f.out
    mask = x.labels != synth.IGNORE_INDEX
    old = kink_free_old(lp, (lp + 0.15 * x.old_noise).astype(np.float32), P["eps_low"],
                        P["eps_high"], mask)
    ref = (lp + 0.3 * x.ref_noise).astype(np.float32)
    pi = np.where(mask, lp, 0.0).reshape(w.n_seq, w.seq_len).sum(axis=1)
    ref_dpo = (pi + (1.5 / P["dpo_beta"]) * x.seq_noise).astype(np.float32)
    ref_kto = (pi + (1.5 / P["kto_beta"]) * x.seq_noise).astype(np.float32)
    losses = {
        "grpo": po.grpo_from_logp(lp, x.labels, w.n_seq, x.advantages, old_logp=old,
                                  ref_logp=ref, beta=P["grpo_beta"], eps_low=P["eps_low"],
                                  eps_high=P["eps_high"]),
        "dpo": po.dpo_from_logp(lp, x.labels, w.n_seq, ref_dpo, beta=P["dpo_beta"]),
        "kto": po.kto_from_logp(lp, x.labels, w.n_seq, ref_kto, x.desirable,
                                kl_ref=P["kl_ref"], beta=P["kto_beta"],
                                desirable_weight=P["desirable_weight"],
                                undesirable_weight=P["undesirable_weight"]),
    }
    tw = synth.Workload(name, T=w.T, H=w.H, V=w.V, chunk_rows=w.chunk_rows, w_std=w.w_std,
                        ignore_count=0, mode="logprob", reduction="none", seed=w.seed,
                        seq_len=w.seq_len, prompt_len=w.prompt_len)
    tokens = sample_tokens(tw, x.labels, rng)
    vocab = sample_vocab(tw, x.labels, tokens, rng)
    edges = vocab_edges(w.V)
    out = dict(tokens=tokens, vocab=vocab, logp=lp[tokens], seed=np.int64(w.seed), old=old,
               ref=ref, ref_dpo=ref_dpo, ref_kto=ref_kto, grad_loss=np.float64(GRAD_LOSS),
               **{k: np.float64(v) for k, v in P.items()})
    for k, r in losses.items():
        c = -GRAD_LOSS * r.dlogp          # log-prob mode: G = -grad_out (P - onehot)
        out[f"{k}_loss"] = np.float64(r.loss)
        out[f"{k}_dh"] = o.grad_hidden_rows(x.hidden, x.weight, x.labels, tokens, c[tokens],
                                            synth.IGNORE_INDEX).astype(np.float32)
        out[f"{k}_dw"] = o.grad_weight_rows(x.hidden, x.weight, x.labels, vocab, c,
                                            f.lse).astype(np.float32)
        out[f"{k}_dw_edge"] = o.grad_weight_rows(x.hidden, x.weight, x.labels, edges, c,
                                                 f.lse)[:, :EDGE_COLS].astype(np.float32)
    out["vocab_edge"] = edges
    path = os.path.join(HERE, f"{name}.npz")
    np.savez(path, **out)
    print(f"{name}: {time.time() - t0:.0f} s -> {path}", flush=True)
    return path


if __name__ == "__main__":
    for n in (sys.argv[1:] or FULL + tuple(VARIANTS) + DISTILL + POLICY):
        if n in DISTILL:
            make_distill(n)
        elif n in POLICY:
            make_policy(n)
        else:
            make(n)
