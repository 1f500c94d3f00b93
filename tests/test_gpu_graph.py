"""The boundary calls under HIP graph capture: cross-entropy forward + backward, the
distillation (KL and JSD) and the GRPO loss with gradients.

The library only launches kernels on the caller's stream (it allocates, clears and
synchronises nothing), so a whole step can be captured once and replayed.
Each replay must reproduce the eager results bit for bit (the kernels are deterministic), also
after new inputs are copied into the captured buffers and with eager work and
synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

from chunked_lm_head_amd import synth
from oracle import flce_oracle as o

import gpu_util as gu

pytestmark = pytest.mark.gpu

T, D, V, CR = 700, 256, 3000, 64


def _inputs(seed):
    return synth.make_inputs(synth.custom("graph", T=T, H=D, V=V, ignore_frac=0.05, seed=seed))


def _graph_case(kind):
    from chunked_lm_head_amd import flce

    dev = gu.device()
    xs = [_inputs(31), _inputs(32)]
    h = gu.bf16_tensor(xs[0].hidden, dev)
    W = gu.bf16_tensor(xs[0].weight, dev)
    y = torch.from_numpy(xs[0].labels).to(dev)
    f32 = dict(dtype=torch.float32, device=dev)
    gm = torch.ones((), **f32)
    g_tok = torch.from_numpy(np.random.default_rng(5).standard_normal(T).astype(np.float32)).to(dev)
    ws = flce.alloc_workspace(T, D, V, CR, dev)
    out, lse, mean = torch.empty(T, **f32), torch.empty(T, **f32), torch.empty((), **f32)
    dh = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((V, D), **f32)
    mode = "nll" if kind == "mean" else "logprob"
    grad = dict(grad_mean=gm) if kind == "mean" else dict(grad_out=g_tok)

    def load(x):
        h.copy_(gu.bf16_tensor(x.hidden, dev))
        W.copy_(gu.bf16_tensor(x.weight, dev))
        y.copy_(torch.from_numpy(x.labels).to(dev))

    def step():
        flce.forward(h, W, y, chunk_rows=CR, mode=mode, workspace=ws, out=out, lse=lse,
                     mean=mean)
        flce.backward(h, W, y, lse, chunk_rows=CR, mode=mode, workspace=ws, grad_hidden=dh,
                      grad_weight=dw, **grad)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (out, lse, mean, dh, dw)]

    refs = []
    for x in xs:  # eager results, which also warm the library up before the capture
        load(x)
        step()
        refs.append(snapshot())

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for i in (0, 1, 0, 1):
        load(xs[i])
        for t in (out, lse, mean, dw):  # poison: every output must be rewritten by the replay
            t.fill_(float("nan"))
        dh.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for name, a, b in zip(("out", "lse", "mean", "dh", "dw"), got, refs[i]):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), \
                (kind, i, name)
    # the two input sets really differ, so the replays recomputed
    assert not torch.equal(refs[0][0], refs[1][0])
    # and the captured step computes the right thing: the oracle on the second input set
    x = xs[1]
    go = g_tok.cpu().numpy() if kind != "mean" else None
    f = o.forward(x.hidden, x.weight, x.labels, synth.IGNORE_INDEX, mode)
    odh, odw = (o.backward(x.hidden, x.weight, x.labels, synth.IGNORE_INDEX, mode, grad_out=go)
                if go is not None else
                o.backward(x.hidden, x.weight, x.labels, synth.IGNORE_INDEX, mode, grad_mean=1.0))
    assert gu.max_abs(refs[1][0].cpu().numpy(), f.out) <= gu.OUT_TOL
    assert gu.rel_fro(refs[1][3].float().cpu().numpy(), odh) <= gu.GRAD_TOL
    assert gu.rel_fro(refs[1][4].cpu().numpy(), odw) <= gu.GRAD_TOL
    del graph


@pytest.mark.parametrize("kind", ["mean", "per_token_logprob"])
def test_captured_step_replays_match_eager(kind):
    print(f"case graph {kind}: T={T} D={D} V={V} chunk_rows={CR}", flush=True)
    _graph_case(kind)


def _replays_match_eager(loads, step, outputs):
    """Eager results for each input set, then one capture of `step` replayed over the sets in
    turn, each replay over poisoned outputs and compared bit for bit."""
    refs = []
    for load in loads:
        load()
        step()
        torch.cuda.synchronize()
        refs.append([t.clone() for t in outputs])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in (0, 1, 0, 1):
        loads[i]()
        for t in outputs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outputs, refs[i])):
            bits = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(a.view(bits), b.view(bits)), (i, j)
    assert not torch.equal(refs[0][0], refs[1][0])
    del graph
    return refs


@pytest.mark.parametrize("divergence", ["kl", "jsd"])
def test_captured_distillation_replays_match_eager(divergence):
    from chunked_lm_head_amd import flce

    dev = gu.device()
    Tn, Ds, Dt, Vn, cr = 520, 128, 192, 2600, 64
    print(f"case graph distill {divergence}: T={Tn} Ds={Ds} Dt={Dt} V={Vn}", flush=True)
    xs = [synth.make_distill_inputs(synth.distill_custom("gd", Tn, Ds, Dt, Vn, chunk_rows=cr,
                                                         ignore_frac=0.05, seed=s))
          for s in (41, 42)]
    bufs = [gu.bf16_tensor(a, dev) for a in (xs[0].s_hidden, xs[0].s_weight, xs[0].t_hidden,
                                              xs[0].t_weight)]
    mask = torch.from_numpy(xs[0].labels).to(dev)
    f32 = dict(dtype=torch.float32, device=dev)
    gm = torch.ones((), **f32)
    kl, mean = torch.empty(Tn, **f32), torch.empty((), **f32)
    dh = torch.empty((Tn, Ds), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((Vn, Ds), **f32)
    ws = torch.empty(flce.distill_workspace_bytes(Tn, Ds, Dt, Vn, cr), dtype=torch.uint8,
                     device=dev)

    def loader(x):
        def load():
            for b, a in zip(bufs, (x.s_hidden, x.s_weight, x.t_hidden, x.t_weight)):
                b.copy_(gu.bf16_tensor(a, dev))
            mask.copy_(torch.from_numpy(x.labels).to(dev))
        return load

    def step():
        flce.distill(*bufs, mask, chunk_rows=cr, grad_mean=gm, grad_hidden=dh, grad_weight=dw,
                     workspace=ws, kl=kl, mean=mean, divergence=divergence, beta=0.5)

    _replays_match_eager([loader(x) for x in xs], step, [kl, mean, dh, dw])


def test_captured_grpo_replays_match_eager():
    from chunked_lm_head_amd import flce

    dev = gu.device()
    n_seq, S, P, Dn, Vn, cr = 3, 200, 40, 128, 2600, 64
    Tn = n_seq * S
    print(f"case graph grpo: n_seq={n_seq} S={S} D={Dn} V={Vn}", flush=True)
    xs = [synth.make_policy_inputs(synth.policy_custom("gp", n_seq, S, P, Dn, Vn, chunk_rows=cr,
                                                       seed=s)) for s in (51, 52)]
    f32 = dict(dtype=torch.float32, device=dev)
    h = gu.bf16_tensor(xs[0].hidden, dev)
    W = gu.bf16_tensor(xs[0].weight, dev)
    y = torch.from_numpy(xs[0].labels).to(dev)
    adv, old, ref = torch.empty(n_seq, **f32), torch.empty(Tn, **f32), torch.empty(Tn, **f32)
    side = []
    for x in xs:  # old and reference log-probs near the policy's own
        lp = flce.forward(gu.bf16_tensor(x.hidden, dev), gu.bf16_tensor(x.weight, dev),
                          torch.from_numpy(x.labels).to(dev), chunk_rows=cr,
                          mode="logprob")[0]
        side.append((torch.from_numpy(x.advantages).to(dev),
                     lp + 0.15 * torch.from_numpy(x.old_noise).to(dev),
                     lp + 0.3 * torch.from_numpy(x.ref_noise).to(dev)))
    gl = torch.ones((), **f32)
    loss, logp = torch.empty((), **f32), torch.empty(Tn, **f32)
    dh = torch.empty((Tn, Dn), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((Vn, Dn), **f32)
    ws = torch.empty(flce.policy_workspace_bytes(Tn, Dn, Vn, cr, n_seq), dtype=torch.uint8,
                     device=dev)

    def loader(i):
        def load():
            h.copy_(gu.bf16_tensor(xs[i].hidden, dev))
            W.copy_(gu.bf16_tensor(xs[i].weight, dev))
            y.copy_(torch.from_numpy(xs[i].labels).to(dev))
            for dst, src in zip((adv, old, ref), side[i]):
                dst.copy_(src)
        return load

    def step():
        flce.grpo_loss(h, W, y, n_seq, adv, old_logp=old, ref_logp=ref, beta=0.04,
                       chunk_rows=cr, grad_loss=gl, grad_hidden=dh, grad_weight=dw,
                       workspace=ws, loss=loss, logp=logp)

    _replays_match_eager([loader(0), loader(1)], step, [logp, loss, dh, dw])
