"""Full-size workloads on the GPU, in the launch configuration bench.py times.

Expected values are oracle outputs for sampled tokens and vocabulary rows,
written by tests/golden/make_golden.py (float64 CPU oracle over all tokens and
the full vocabulary).  Beyond the samples, properties that hold at any size
are checked on the complete outputs:
  * each row of G sums to zero, so the vocabulary sum of dW vanishes (not with
    a softcap, whose derivative differs from logit to logit);
  * <dH, H> = <dW, W> (both equal sum_tv G_tv z_tv);
  * ignored tokens and tokens with zero upstream grad have exactly zero dH rows
    (and ignored tokens output exactly 0).
"""
import math
import os

import numpy as np
import pytest
import torch

from chunked_lm_head_amd import synth

import gpu_util as gu

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
# golden file -> workload; the transform variants store their transform in the file
NAMES = ["single_chunk", "qwen3_8b_sft", "grpo_logprob", "long_context",
         "single_chunk_scaled", "qwen3_8b_sft_softcap"]


def _golden(name):
    path = os.path.join(HERE, "golden", f"{name}.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}; run tests/golden/make_golden.py")
    return np.load(path)


def check_edge_rows(dw, g, key="dw_edge"):
    """dW rows on both sides of every vocabulary chunk edge (first columns kept by the
    golden script), each within the gradient tolerance on its own."""
    edges = torch.from_numpy(g["vocab_edge"]).to(dw.device)
    want = g[key].astype(np.float64)
    got = dw[edges][:, :want.shape[1]].cpu().numpy()
    worst = max(gu.rel_fro(got[i], want[i]) for i in range(len(want)))
    print(f"  {len(want)} chunk-edge dW rows: worst row rel {worst:.2e}", flush=True)
    assert worst <= gu.GRAD_TOL, worst


def _run_full(name, transform=None):
    from chunked_lm_head_amd import flce

    w = synth.WORKLOADS[name]
    xf = gu.binding_transform(transform)
    print(f"case {name}: T={w.T} D={w.H} V={w.V} chunk_rows={w.chunk_rows} transform {xf}",
          flush=True)
    x = synth.make_inputs(w)
    dev = gu.device()
    h = gu.bf16_tensor(x.hidden, dev)
    W = gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    ws = flce.alloc_workspace(w.T, w.H, w.V, w.chunk_rows, dev)
    out, lse, mean = flce.forward(h, W, y, chunk_rows=w.chunk_rows, mode=w.mode, transform=xf,
                                  workspace=ws)
    if x.grad_out is not None:
        kw = dict(grad_out=torch.from_numpy(x.grad_out).to(dev))
    else:
        kw = dict(grad_mean=torch.ones((), dtype=torch.float32, device=dev))
    dh, dw = flce.backward(h, W, y, lse, chunk_rows=w.chunk_rows, mode=w.mode, transform=xf,
                           workspace=ws, **kw)
    torch.cuda.synchronize()
    return w, x, h, W, out, lse, mean, dh, dw


@pytest.mark.parametrize("name", NAMES)
def test_full_size_against_oracle_samples(name):
    g = _golden(name)
    base = str(g["workload"]) if "workload" in g else name
    tr = g["transform"] if "transform" in g else None
    w, x, h, W, out, lse, mean, dh, dw = _run_full(base, tr)
    assert int(g["seed"]) == w.seed
    tok = torch.from_numpy(g["tokens"]).to(h.device)
    voc = torch.from_numpy(g["vocab"]).to(h.device)
    out_s = out[tok].cpu().numpy()
    lse_s = lse[tok].cpu().numpy()
    assert gu.max_abs(out_s, g["out"]) <= gu.OUT_TOL, gu.max_abs(out_s, g["out"])
    assert gu.max_abs(lse_s, g["lse"]) <= gu.OUT_TOL, gu.max_abs(lse_s, g["lse"])
    assert abs(float(mean.cpu()) - float(g["mean"])) <= gu.OUT_TOL
    dh_s = dh[tok].float().cpu().numpy()
    dw_s = dw[voc].cpu().numpy()
    e_dh = gu.rel_fro(dh_s, g["dh"].astype(np.float64))
    e_dw = gu.rel_fro(dw_s, g["dw"].astype(np.float64))
    print(f"{name}: |d out| {gu.max_abs(out_s, g['out']):.2e} |d lse| "
          f"{gu.max_abs(lse_s, g['lse']):.2e} |d mean| {abs(float(mean.cpu()) - float(g['mean'])):.2e}"
          f" dH rel {e_dh:.2e} dW rel {e_dw:.2e}", flush=True)
    assert e_dh <= gu.GRAD_TOL, e_dh
    assert e_dw <= gu.GRAD_TOL, e_dw
    check_edge_rows(dw, g)

    # properties on the complete outputs (fp64 reductions on the GPU)
    dw64 = dw.double()
    if tr is None or float(tr[2]) == 0.0:
        # rows of G sum to zero unless a softcap makes dz'/dz vary along the row
        col = dw64.sum(dim=0)
        fro = torch.linalg.norm(dw64)
        assert float(torch.linalg.norm(col) / fro) <= 1e-2
    lhs = float((dh.double() * h.double()).sum())
    rhs = float((dw64 * W.double()).sum())
    assert abs(lhs - rhs) <= 1e-2 * max(abs(lhs), abs(rhs), 1e-30), (lhs, rhs)
    yl = torch.from_numpy(x.labels).to(h.device)
    ign = yl == synth.IGNORE_INDEX
    if bool(ign.any()):
        assert bool((out[ign] == 0).all())
        assert bool((dh[ign] == 0).all())
    if x.grad_out is not None:
        zero = torch.from_numpy(x.grad_out == 0).to(h.device)
        assert bool((dh[zero] == 0).all())
    assert bool(torch.isfinite(out[~ign]).all())


def workspace_bound(T, D, V, chunk_rows):
    """Device memory the cross-entropy step may need beyond its inputs and outputs, from the
    shape alone: one bf16 gradient block within the fp32 logits of one chunk
    (chunk_rows * V * 4), the fp32 dH sums of a row block of at most 8,192 rows (split-K
    copies capped at 128 MiB), the transposed bf16 hidden states of that row block, and
    per-token terms (forward partials of about 4 MiB, six fp32 values per token)."""
    r_max = min(8192, -(-T // 256) * 256)
    return (chunk_rows * V * 4 + max(r_max * D * 4, 128 << 20) + r_max * D * 2
            + 24 * T + (8 << 20))


def test_long_context_memory_stays_within_the_workspace_formula():
    """Peak device memory beyond inputs and outputs obeys workspace_bound: one chunk of fp32
    logits plus terms linear in D and in T, never anything of size T x V."""
    from chunked_lm_head_amd import flce

    w = synth.WORKLOADS["long_context"]
    bound = workspace_bound(w.T, w.H, w.V, w.chunk_rows)
    assert bound < w.T * w.V * 4 / 100           # full fp32 logits: 79.7 GB
    assert flce.workspace_bytes(w.T, w.H, w.V, w.chunk_rows) <= bound
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    _, _, h, W, out, lse, mean, dh, dw = _run_full("long_context")
    peak = torch.cuda.max_memory_allocated() - base
    io = sum(t.numel() * t.element_size() for t in (h, W, out, lse, mean, dh, dw))
    io += w.T * 8  # labels
    assert peak - io <= bound, (peak, io, bound)


@pytest.mark.parametrize("name", ["distill_qwen3", "distill_qwen3_jsd"])
def test_distill_full_size_against_oracle_samples(name):
    """Distillation at the student-8B / wider-teacher shape, KL and JSD: sampled per-token
    divergence, the mean, and sampled dH / dW rows of the student (float64 oracle over
    all tokens and the full vocabulary, tests/golden/make_golden.py)."""
    from chunked_lm_head_amd import flce

    g = _golden(name)
    w = synth.DISTILL_WORKLOADS["distill_qwen3"]
    assert int(g["seed"]) == w.seed
    divergence = str(g["divergence"]) if "divergence" in g else "kl"
    beta = float(g["beta"]) if "beta" in g else 0.5
    print(f"case {name}: T={w.T} Ds={w.Hs} Dt={w.Ht} V={w.V} {divergence} beta {beta}",
          flush=True)
    x = synth.make_distill_inputs(w)
    dev = gu.device()
    sh, sw = gu.bf16_tensor(x.s_hidden, dev), gu.bf16_tensor(x.s_weight, dev)
    th, tw = gu.bf16_tensor(x.t_hidden, dev), gu.bf16_tensor(x.t_weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    kl, mean, dh, dw = flce.distill(sh, sw, th, tw, y, chunk_rows=w.chunk_rows,
                                    grad_mean=torch.ones((), dtype=torch.float32, device=dev),
                                    divergence=divergence, beta=beta)
    torch.cuda.synchronize()
    tok = torch.from_numpy(g["tokens"]).to(dev)
    voc = torch.from_numpy(g["vocab"]).to(dev)
    kl_s = kl[tok].cpu().numpy()
    e = (gu.max_abs(kl_s, g["kl"]), abs(float(mean.cpu()) - float(g["mean"])),
         gu.rel_fro(dh[tok].float().cpu().numpy(), g["dh"].astype(np.float64)),
         gu.rel_fro(dw[voc].cpu().numpy(), g["dw"].astype(np.float64)))
    print(f"{name}: |d value| {e[0]:.2e} |d mean| {e[1]:.2e} dH rel {e[2]:.2e} "
          f"dW rel {e[3]:.2e}", flush=True)
    assert e[0] <= gu.OUT_TOL and e[1] <= gu.OUT_TOL, e
    assert e[2] <= gu.GRAD_TOL and e[3] <= gu.GRAD_TOL, e
    check_edge_rows(dw, g)
    # properties on the complete outputs: the divergence >= 0 (up to rounding; the JSD
    # also <= ln 2 at beta = 1/2), masked tokens are 0
    m = y == synth.IGNORE_INDEX
    assert bool((kl[m] == 0).all()) and bool((dh[m] == 0).all())
    assert float(kl[~m].min()) > -1e-3
    if divergence == "jsd" and beta == 0.5:
        assert float(kl.max()) <= math.log(2.0) + 1e-3
    lhs = float((dh.double() * sh.double()).sum())
    rhs = float((dw.double() * sw.double()).sum())
    assert abs(lhs - rhs) <= 1e-2 * max(abs(lhs), abs(rhs), 1e-30), (lhs, rhs)


_POLICY = {}


def _policy_inputs():
    if not _POLICY:
        w = synth.POLICY_WORKLOADS["grpo_qwen3"]
        _POLICY.update(w=w, x=synth.make_policy_inputs(w))
    return _POLICY["w"], _POLICY["x"]


@pytest.mark.parametrize("kind", ["grpo", "dpo", "kto"])
def test_policy_full_size_against_oracle_samples(kind):
    """GRPO, DPO and KTO at the GRPO example's size (4 sequences of 8,192 tokens, 1,024 of
    them prompt, hidden 4,096, vocabulary 128,000); old / reference log-probs and reference
    sequence log-probs are stored with the oracle values (built from the oracle's own
    log-probs by the golden script)."""
    from chunked_lm_head_amd import flce

    g = _golden("grpo_qwen3")
    w, x = _policy_inputs()
    assert int(g["seed"]) == w.seed
    print(f"case grpo_qwen3 {kind}: T={w.T} D={w.H} V={w.V} sequences {w.n_seq}", flush=True)
    dev = gu.device()
    h = gu.bf16_tensor(x.hidden, dev)
    W = gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    ws = torch.empty(flce.policy_workspace_bytes(w.T, w.H, w.V, w.chunk_rows, w.n_seq),
                     dtype=torch.uint8, device=dev)
    common = dict(chunk_rows=w.chunk_rows, workspace=ws,
                  grad_loss=torch.tensor(float(g["grad_loss"]), dtype=torch.float32, device=dev),
                  logp=torch.empty(w.T, dtype=torch.float32, device=dev))
    if kind == "grpo":
        out = flce.grpo_loss(h, W, y, w.n_seq, t(x.advantages), old_logp=t(g["old"]),
                             ref_logp=t(g["ref"]), beta=float(g["grpo_beta"]),
                             eps_low=float(g["eps_low"]), eps_high=float(g["eps_high"]), **common)
    elif kind == "dpo":
        out = flce.dpo_loss(h, W, y, w.n_seq, t(g["ref_dpo"]), beta=float(g["dpo_beta"]),
                            **common)
    else:
        out = flce.kto_loss(h, W, y, w.n_seq, t(g["ref_kto"]), t(x.desirable),
                            kl_ref=torch.tensor(float(g["kl_ref"]), dtype=torch.float32,
                                                device=dev),
                            beta=float(g["kto_beta"]),
                            desirable_weight=float(g["desirable_weight"]),
                            undesirable_weight=float(g["undesirable_weight"]), **common)
    torch.cuda.synchronize()
    loss, logp, dh, dw = out
    tok = torch.from_numpy(g["tokens"]).to(dev)
    voc = torch.from_numpy(g["vocab"]).to(dev)
    e = (abs(float(loss.cpu()) - float(g[f"{kind}_loss"])),
         gu.max_abs(logp[tok].cpu().numpy(), g["logp"]),
         gu.rel_fro(dh[tok].float().cpu().numpy(), g[f"{kind}_dh"].astype(np.float64)),
         gu.rel_fro(dw[voc].cpu().numpy(), g[f"{kind}_dw"].astype(np.float64)))
    print(f"  loss {float(loss.cpu()):.6f} (oracle {float(g[f'{kind}_loss']):.6f}) |d loss| "
          f"{e[0]:.2e} |d logp| {e[1]:.2e} dH rel {e[2]:.2e} dW rel {e[3]:.2e}", flush=True)
    assert e[0] <= gu.OUT_TOL and e[1] <= gu.OUT_TOL, e
    assert e[2] <= gu.GRAD_TOL and e[3] <= gu.GRAD_TOL, e
    check_edge_rows(dw, g, f"{kind}_dw_edge")
    # properties on the complete outputs
    lhs = float((dh.double() * h.double()).sum())
    rhs = float((dw.double() * W.double()).sum())
    assert abs(lhs - rhs) <= 1e-2 * max(abs(lhs), abs(rhs), 1e-30), (lhs, rhs)
    prompt = y == synth.IGNORE_INDEX
    assert bool((dh[prompt] == 0).all()) and bool((logp[prompt] == 0).all())
    assert bool(torch.isfinite(logp).all())
