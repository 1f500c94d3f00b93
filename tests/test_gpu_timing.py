"""Per-launch kernel timing: with timing on, the library reports every kernel it launched,
in launch order and with positive durations, and computes exactly what it computes with
timing off."""
import pytest
import torch

from chunked_lm_head_amd import synth

import gpu_util as gu

pytestmark = pytest.mark.gpu


def _expected_ce(plan, with_mean=True):
    names = (["fwd_lse", "fwd_combine"] + (["fwd_mean"] if with_mean else [])
             + ["bwd_prep", "bwd_zero_rows"])
    for _ in range(plan["row_blocks"]):
        names.append("bwd_ht")
        names += ["bwd_grad", "bwd_dh", "bwd_dw"] * plan["vocab_chunks"]
        names.append("bwd_dh_out")
    return names


def test_timing_lists_every_launch_and_changes_nothing():
    from chunked_lm_head_amd import flce

    w = synth.custom("timing", T=1300, H=264, V=3100, chunk_rows=32, ignore_frac=0.05, seed=81)
    x = synth.make_inputs(w)
    dev = gu.device()
    h, W = gu.bf16_tensor(x.hidden, dev), gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    cr = w.chunk_rows
    g = torch.tensor(0.9, dtype=torch.float32, device=dev)

    def run():
        out, lse, mean = flce.forward(h, W, y, chunk_rows=cr)
        dh, dw = flce.backward(h, W, y, lse, grad_mean=g, chunk_rows=cr)
        return out, lse, mean, dh, dw

    ref = run()
    torch.cuda.synchronize()
    plan = flce.describe_plan(w.T, w.H, w.V, cr)
    assert plan["row_blocks"] >= 1 and plan["vocab_chunks"] >= 2, plan
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flce.timing_begin(4096)
    with pytest.raises(flce.FlceError):
        flce.timing_begin(16)                      # already on
    a.record()
    got = run()
    b.record()
    rows, n, dropped = flce.timing_end(4096)
    torch.cuda.synchronize()
    for r, t in zip(ref, got):
        assert torch.equal(r, t)
    names = [k for k, _ in rows]
    assert names == _expected_ce(plan), names
    assert n == len(rows) and dropped == 0
    assert all(ms > 0 for _, ms in rows), rows
    total, outer = sum(ms for _, ms in rows), a.elapsed_time(b)
    print(f"  {n} launches, {total:.3f} ms in kernels, {outer:.3f} ms between outer events",
          flush=True)
    # the intervals tile the span of the two calls (the gap between the calls aside)
    assert total <= outer * 1.001 + 0.05, (total, outer)
    # timing is off again: nothing more is recorded
    with pytest.raises(flce.FlceError):
        flce.timing_end(16)


def test_timing_drops_marks_past_its_capacity():
    from chunked_lm_head_amd import flce

    w = synth.custom("timing_small", T=300, H=128, V=900, chunk_rows=16, ignore_frac=0.0,
                     seed=82)
    x = synth.make_inputs(w)
    dev = gu.device()
    h, W = gu.bf16_tensor(x.hidden, dev), gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    flce.timing_begin(3)                           # the start mark + two kernels
    flce.forward(h, W, y, chunk_rows=w.chunk_rows)
    rows, n, dropped = flce.timing_end(8)
    assert [k for k, _ in rows] == ["fwd_lse", "fwd_combine"] and n == 2
    assert dropped == 1                            # fwd_mean's mark found no event
    assert all(ms > 0 for _, ms in rows)


def test_timing_of_distillation_names_its_block_kernels():
    from chunked_lm_head_amd import flce

    w = synth.distill_custom("timing_distill", T=600, Hs=128, Ht=192, V=2100, ws_std=0.3,
                             wt_std=0.3, ignore_frac=0.1, reduction="mean", seed=83)
    x = synth.make_distill_inputs(w)
    dev = gu.device()
    sh, sw = gu.bf16_tensor(x.s_hidden, dev), gu.bf16_tensor(x.s_weight, dev)
    th, tw = gu.bf16_tensor(x.t_hidden, dev), gu.bf16_tensor(x.t_weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    one = torch.ones((), dtype=torch.float32, device=dev)
    kw = dict(chunk_rows=w.chunk_rows, grad_mean=one)
    ref = flce.distill(sh, sw, th, tw, y, **kw)
    flce.timing_begin(4096)
    got = flce.distill(sh, sw, th, tw, y, **kw)
    rows, n, dropped = flce.timing_end(4096)
    torch.cuda.synchronize()
    for r, t in zip(ref, got):
        assert torch.equal(r, t)
    names = [k for k, _ in rows]
    assert dropped == 0 and names[:4] == ["fwd_lse", "dst_lse", "fwd_lse", "dst_lse"], names
    blocks = names.count("dst_teacher")
    assert blocks >= 2 and names.count("dst_student") == blocks
    assert names.count("dst_dh") == blocks and names.count("dst_dw") == blocks
    assert names[-2:] == ["dst_combine", "fwd_mean"], names
    assert all(ms > 0 for _, ms in rows)


def test_timing_of_a_policy_loss_and_the_allocation_free_forward():
    from chunked_lm_head_amd import flce

    w = synth.policy_custom("timing_policy", n_seq=2, seq_len=384, prompt_len=64, H=128, V=1900,
                            seed=84)
    x = synth.make_policy_inputs(w)
    dev = gu.device()
    h, W = gu.bf16_tensor(x.hidden, dev), gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    adv = torch.from_numpy(x.advantages).to(dev)
    one = torch.ones((), dtype=torch.float32, device=dev)
    ref = flce.grpo_loss(h, W, y, w.n_seq, adv, beta=0.0, chunk_rows=w.chunk_rows,
                         grad_loss=one)
    out = torch.empty(w.T, dtype=torch.float32, device=dev)
    lse = torch.empty(w.T, dtype=torch.float32, device=dev)
    flce.timing_begin(4096)
    got = flce.grpo_loss(h, W, y, w.n_seq, adv, beta=0.0, chunk_rows=w.chunk_rows,
                         grad_loss=one)
    flce.forward_noalloc(h, W, y, chunk_rows=w.chunk_rows, out=out, lse=lse)
    rows, n, dropped = flce.timing_end(4096)
    torch.cuda.synchronize()
    for r, t in zip(ref, got):
        assert (r is None and t is None) or torch.equal(r, t)
    names = [k for k, _ in rows]
    plan = flce.describe_plan(w.T, w.H, w.V, w.chunk_rows)
    # the tile list and log-prob forward, the loss kernels, the log-prob backward, then the
    # second forward
    want = (["fwd_skip_prep", "fwd_lse", "fwd_combine", "policy", "bwd_prep", "bwd_zero_rows"]
            + (["bwd_ht"] + ["bwd_grad", "bwd_dh", "bwd_dw"] * plan["vocab_chunks"]
               + ["bwd_dh_out"]) * plan["row_blocks"]
            + ["fwd_lse", "fwd_combine"])
    assert dropped == 0 and names == want, names
    assert all(ms > 0 for _, ms in rows)
