"""Throughput of the chunked LM-head + cross-entropy forward + backward on one MI355X.

One step = flce_forward + flce_backward (mean NLL, upstream grad 1) over the
whole synthetic batch, inputs resident in HBM, workspace preallocated.  Work
per step is 8*T*V*D FLOPs: the logit GEMM (2TVD), its recompute in the backward
(2TVD), dH = G W (2TVD) and dW = G^T H (2TVD).  The backward skips 256-token tiles
in which no token has a gradient (prompt tokens of a policy loss, a per-token upstream
gradient that is zero); the FLOPs reported are the ones the kernels execute.

Prints one JSON line.  ``roofline`` describes the GEMM kernel with the most time
per step (the fused forward, the recompute, dH or dW), timed with the HIP events
the library records after each kernel on the stream it runs on (instrumented steps
after the timed ones), and lists all four under ``kernels``; ``cpu_baseline``
times the float64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LM-head+CE fwd+bwd tokens/s & % bf16 MFMA peak (H=4096, V=151,936)"
PEAK_BF16 = 2.5e15          # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12           # MI355X HBM3E, B/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b_sft")
    ap.add_argument("--loss", choices=("grpo", "dpo", "kto"), default="grpo",
                    help="policy loss of a policy workload (grpo_qwen3)")
    ap.add_argument("--divergence", choices=("kl", "jsd"), default="kl",
                    help="divergence of a distillation workload")
    ap.add_argument("--beta", type=float, default=0.5,
                    help="JSD weight of the teacher in the mixture (--divergence jsd)")
    ap.add_argument("--chunk-rows", type=int, default=None)
    ap.add_argument("--token-shard", type=int, default=1, metavar="N",
                    help="run one GPU's share of a token-parallel split over N GPUs: the "
                         "cross-entropy workload with T / N of its tokens")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--cpu-sample-vocab", type=int, default=1 << 30)
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="only time the vendor GEMM (torch.mm -> hipBLASLt) at this path's shapes")
    ap.add_argument("--sample-power", action="store_true",
                    help="sample socket power and GFX clocks with amd-smi during the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (reference for HBM counters)")
    ap.add_argument("--logit-scale-multiply", type=float, default=0.0,
                    help="logit transform: multiply each logit (0 = off)")
    ap.add_argument("--logit-scale-divide", type=float, default=0.0,
                    help="logit transform: divide each logit (0 = off)")
    ap.add_argument("--logit-softcapping", type=float, default=0.0,
                    help="logit transform: cap * tanh(z / cap) (0 = off)")
    ap.add_argument("--temperature", type=float, default=1.0,
                    help="logit transform: divide by the temperature, last")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch from rocprofv3 counters (optional)")
    return ap.parse_args()


def cpu_baseline(x, n_tokens: int, n_vocab: int, transform=None) -> dict:
    """The oracle, untouched, on a bounded sample: the first n_tokens tokens (about 20 s of
    host work at the defaults) against the whole vocabulary, or against its first n_vocab
    rows with the labels folded into that range; the oracle's work is linear in the
    vocabulary, so a partial sample's rate is scaled by n_vocab / V."""
    import numpy as np

    from oracle import flce_oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    V = x.weight.shape[0]
    n_vocab = min(n_vocab, V)
    h = x.hidden[:n_tokens]
    wt = x.weight[:n_vocab]
    y = x.labels[:n_tokens].copy()
    used = y != -100
    y[used] %= n_vocab
    t0 = time.perf_counter()
    tr = flce_oracle.LogitTransform(**transform) if transform else None
    f = flce_oracle.forward(h, wt, y, transform=tr)
    flce_oracle.backward(h, wt, y, lse=f.lse, grad_mean=1.0, transform=tr)
    dt = time.perf_counter() - t0
    vocab = (f"all {V} vocabulary rows" if n_vocab == V else
             f"the first {n_vocab} of {V} vocabulary rows (labels folded into the slice; "
             f"rate scaled by {n_vocab}/{V})")
    return {"value": round(n_tokens / dt * n_vocab / V, 3), "unit": "tokens/s",
            "cores": int(cores), "kind": "oracle",
            "sample": f"first {n_tokens} tokens x {vocab}, float64 numpy forward + backward "
                      f"in {dt:.1f} s"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the design notes describe how it would shard).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 64 << 20  # fp32 elements: 256 MiB read + 256 MiB written per copy
        a = torch.ones(n, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "copies": 3}))
        return

    from chunked_lm_head_amd import flce, synth

    if args.gemm_ceiling:
        gemm_ceiling(synth.WORKLOADS[args.workload])
        return

    if args.token_shard != 1 and args.workload not in synth.WORKLOADS:
        raise SystemExit("--token-shard applies to the cross-entropy workloads only")
    if args.workload in synth.DISTILL_WORKLOADS:
        distill_main(args)
        return
    if args.workload in synth.POLICY_WORKLOADS:
        policy_main(args)
        return
    w = synth.WORKLOADS[args.workload]
    if args.token_shard != 1:
        n = args.token_shard
        if n < 1 or w.T % n or (w.seq_len and (w.T // n) % w.seq_len):
            raise SystemExit(f"--token-shard {n} does not split {w.name}'s {w.T} tokens into "
                             "equal shards of whole sequences")
        w = dataclasses.replace(w, T=w.T // n,
                                ignore_count=int(round(w.ignore_count / n)))
    chunk_rows = args.chunk_rows or w.chunk_rows
    xf_vals = dict(scale_multiply=args.logit_scale_multiply, scale_divide=args.logit_scale_divide,
                   softcap=args.logit_softcapping, temperature=args.temperature)
    has_xf = xf_vals != dict(scale_multiply=0.0, scale_divide=0.0, softcap=0.0, temperature=1.0)
    xf = dict(logit_scale_multiply=args.logit_scale_multiply,
              logit_scale_divide=args.logit_scale_divide,
              logit_softcapping=args.logit_softcapping, temperature=args.temperature)
    t_gen = time.perf_counter()
    x = synth.make_inputs(w)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    h = torch.from_numpy(x.hidden.view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(x.weight.view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.from_numpy(x.labels).to(dev)
    T, D, V = w.T, w.H, w.V
    ws = flce.alloc_workspace(T, D, V, chunk_rows, dev)
    out = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    mean = torch.empty((), dtype=torch.float32, device=dev)
    dh = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((V, D), dtype=torch.float32, device=dev)
    gmean = torch.ones((), dtype=torch.float32, device=dev)
    gout = None
    if w.reduction == "none":
        gout = torch.from_numpy(x.grad_out).to(dev)
    gkw = dict(grad_out=gout) if gout is not None else dict(grad_mean=gmean)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        flce.forward(h, W, y, chunk_rows=chunk_rows, mode=w.mode, transform=xf, workspace=ws,
                     out=out, lse=lse, mean=mean)
        if ev is not None:
            ev[1].record()
        flce.backward(h, W, y, lse, chunk_rows=chunk_rows, mode=w.mode, transform=xf,
                      grad_hidden=dh, grad_weight=dw, workspace=ws, **gkw)
        if ev is not None:
            ev[2].record()

    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # device memory the step needs beyond its resident inputs and outputs: the workspace
    peak_extra = torch.cuda.max_memory_allocated(dev) - base_alloc + ws.numel()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sampler = PowerSampler() if args.sample_power else None
    torch.cuda.synchronize()
    if sampler:
        sampler.start()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    power = sampler.stop() if sampler else None
    total_ms = start.elapsed_time(end)
    ms = total_ms / args.steps
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    bwd_avg = sum(bwd_ms) / len(bwd_ms)
    step_ms = sorted(f + b for f, b in zip(fwd_ms, bwd_ms))
    median_ms = step_ms[len(step_ms) // 2]
    tokens_per_s = T / (ms / 1e3)
    fwd_flops = 2.0 * T * V * D
    plan = flce.describe_plan(T, D, V, chunk_rows)
    active = x.labels != synth.IGNORE_INDEX
    if x.grad_out is not None:
        active &= x.grad_out != 0
    bwd = backward_flops(active, plan["row_block"], V, D)
    gemm_flops = {"fwd_lse": fwd_flops, **{k: bwd[k] for k in ("bwd_grad", "bwd_dh", "bwd_dw")}}
    step_flops = sum(gemm_flops.values())

    # Per-kernel times of the four GEMM kernels, outside the timed region: the library's
    # per-launch events over instrumented steps (one event on the stream after each
    # kernel it launches).  Each GEMM kernel does 2TVD per step, less the skipped tiles.
    kernels, inst = kernel_breakdown(step, max(3, min(args.steps, 10)), gemm_flops)
    traffic = load_traffic(args) if (args.logit_softcapping == 0.0
                                     and args.token_shard == 1) else {}
    # Algorithmic HBM bytes per step of each GEMM kernel (each operand and output once per
    # launch that needs it; the plan's row blocks n_rb and vocabulary chunks n_vc):
    #   forward:   H and W once, labels, two fp32 values per token out;
    #   recompute: per (row block, chunk) its H rows and W rows, the bf16 G block written;
    #   dH:        G read, W rows per row block, fp32 dH sums written (read back after
    #              the first chunk);
    #   dW:        G read, H^T per chunk, fp32 dW written (read back after the first block).
    n_rb, n_vc = plan["row_blocks"], plan["vocab_chunks"]
    step_bytes = {
        "fwd_lse": 2.0 * T * D + 2.0 * V * D + 8.0 * T + 8.0 * T,
        "bwd_grad": 2.0 * n_vc * T * D + 2.0 * n_rb * V * D + 2.0 * T * V,
        "bwd_dh": 2.0 * T * V + 2.0 * n_rb * V * D + 4.0 * T * D * (2 * n_vc - 1),
        "bwd_dw": 2.0 * T * V + 2.0 * n_vc * T * D + 4.0 * V * D * (2 * n_rb - 1),
    }
    for k, rec in kernels.items():
        rec["traffic"] = traffic.get(k, {}).get("hbm_bytes_per_launch")
        n = rec["launches_per_step"]
        rec["algorithmic_bytes_per_launch"] = step_bytes[k] / n
        # below the ridge (peak FLOP/s over peak B/s) a kernel is HBM-bound
        if gemm_flops[k] / step_bytes[k] < PEAK_BF16 / PEAK_HBM:
            rate = step_bytes[k] / (rec["ms_per_step"] / 1e3)
            rec.update(bound="hbm", achieved_gbps=round(rate / 1e9, 1),
                       frac_hbm=round(rate / PEAK_HBM, 4))
        else:
            rec["bound"] = "mfma"
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    if kernels[dom]["bound"] == "hbm":
        roofline = {"kernel": dom, "bound": "hbm", "achieved": kernels[dom]["achieved_gbps"],
                    "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": kernels[dom]["frac_hbm"],
                    "algorithmic_bytes_per_launch": kernels[dom]["algorithmic_bytes_per_launch"]}
    else:
        roofline = {"kernel": dom, "bound": "mfma", "achieved": kernels[dom]["achieved"],
                    "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                    "frac": kernels[dom]["frac"]}
    roofline.update({
        "traffic": kernels[dom]["traffic"],
        "algorithmic_flops_per_launch": kernels[dom]["algorithmic_flops_per_launch"],
        "launches_per_step": kernels[dom]["launches_per_step"],
        "avg_launch_us": kernels[dom]["avg_launch_us"],
        "kernels": kernels,
        "instrumented": inst,
        "note": "the GEMM kernel with the most time per step; per-launch durations from "
                "events the library records after each kernel on its stream, over "
                "instrumented steps run after the timed ones",
    })

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "hidden": D, "vocab": V,
                   **({"token_shard": f"1/{args.token_shard}"} if args.token_shard != 1
                      else {}),
                   "chunk_rows": chunk_rows, "mode": w.mode, "reduction": w.reduction,
                   "ignored_tokens": w.ignore_count,
                   **({"logit_transform": xf_vals} if has_xf else {})},
        "mfma_frac_of_step": round(step_flops / (ms / 1e3) / PEAK_BF16, 4),
        "executed_flops_per_step": step_flops,
        "skipped_token_tiles": f"{bwd['skipped_token_tiles']} of {bwd['token_tiles']}",
        "ms_per_step_median": round(median_ms, 4),
        "fwd_ms": round(fwd_avg, 4),
        "bwd_ms": round(bwd_avg, 4),
        "workspace_bytes": int(ws.numel()),
        "peak_extra_bytes": int(peak_extra),
        "roofline": roofline,
    }
    if power is not None:
        line["power"] = power
    print(f"[bench] {args.workload}: inputs drawn in {t_gen:.1f} s; step {ms:.3f} ms "
          f"(fwd {fwd_avg:.3f}, bwd {bwd_avg:.3f})", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, min(args.cpu_sample_tokens, T),
                                           args.cpu_sample_vocab, xf_vals if has_xf else None)
    print(json.dumps(line), flush=True)


def backward_flops(active, row_block: int, V: int, D: int) -> dict:
    """FLOPs per step that the three backward GEMM kernels execute, given which tokens
    carry a gradient (a label that is not ignored and a non-zero upstream gradient).  A
    256-token tile without any such token is left out of the recompute, dH and dW: the
    tiles with a gradient are packed into the leading row blocks.  With every tile active
    each kernel does 2TVD.  (row_block is the planner's, kept for the caller's record.)"""
    import numpy as np

    T = int(active.shape[0])
    n_t = -(-T // 256)
    pad = np.zeros(n_t * 256, dtype=bool)
    pad[:T] = active
    tile_any = pad.reshape(n_t, 256).any(axis=1)
    tile_tokens = np.minimum(256, T - 256 * np.arange(n_t))
    gd = int(tile_tokens[tile_any].sum())
    f = 2.0 * V * D * gd
    return {"bwd_grad": f, "bwd_dh": f, "bwd_dw": f,
            "skipped_token_tiles": int(n_t - tile_any.sum()), "token_tiles": int(n_t),
            "row_block": int(row_block)}


def kernel_breakdown(step, steps: int, flops: dict) -> tuple:
    """Per-kernel times over `steps` calls of step() with the library's per-launch timing
    on (an event on the stream after every kernel it launches), outside the timed region.
    flops maps kernel names to algorithmic FLOPs per step; returns ({kernel: launches per
    step, ms per step, average launch duration, achieved rate and fraction of peak}, the
    instrumented steps' own time and the sum of all kernels' times per step)."""
    import torch

    from chunked_lm_head_amd import flce

    cap = 1 << 15
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flce.timing_begin(cap)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    rows, n, dropped = flce.timing_end(cap)
    torch.cuda.synchronize()
    if dropped or n > cap or any(ms < 0 for _, ms in rows):
        raise RuntimeError(f"kernel timing incomplete: {n} launches, {dropped} marks dropped")
    per = {}
    for k, ms in rows:
        per.setdefault(k, []).append(ms)
    kernels = {}
    for k, f in flops.items():
        v = per.get(k)
        if not v:
            continue
        t = sum(v) / steps
        kernels[k] = {"launches_per_step": len(v) / steps, "ms_per_step": round(t, 4),
                      "avg_launch_us": round(sum(v) / len(v) * 1e3, 1),
                      "achieved": round(f / (t / 1e3) / 1e12, 2),
                      "frac": round(f / (t / 1e3) / PEAK_BF16, 4),
                      "algorithmic_flops_per_launch": f * steps / len(v)}
    inst = {"steps": steps, "ms_per_step": round(a.elapsed_time(b) / steps, 4),
            "kernel_ms_per_step": round(sum(ms for _, ms in rows) / steps, 4)}
    return kernels, inst


def load_traffic(args) -> dict:
    """Per-kernel HBM bytes per launch from profiles/traffic.json, for the kernels whose
    record was measured on the current kernel sources (a hash of the three files)."""
    try:
        tj = json.load(open(args.traffic_json)).get(args.workload, {})
    except Exception:
        return {}
    sha = _kernel_sha()
    return {k: v for k, v in tj.items() if isinstance(v, dict) and v.get("source_sha") == sha}


def distill_main(args) -> None:
    """One step = one flce_distill call with the mean's gradients: both heads'
    log-sum-exps, then per block the teacher's probabilities and the student's
    gradient, dH and dW.  Work: teacher 2 x 2TVDt, student 4 x 2TVDs FLOPs."""
    import numpy as np
    import torch

    from chunked_lm_head_amd import flce, synth

    w = synth.DISTILL_WORKLOADS[args.workload]
    chunk_rows = args.chunk_rows or w.chunk_rows
    xf = dict(logit_scale_multiply=args.logit_scale_multiply,
              logit_scale_divide=args.logit_scale_divide,
              logit_softcapping=args.logit_softcapping, temperature=args.temperature)
    t_gen = time.perf_counter()
    x = synth.make_distill_inputs(w)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    sh, sw, th, tw = bf16(x.s_hidden), bf16(x.s_weight), bf16(x.t_hidden), bf16(x.t_weight)
    y = torch.from_numpy(x.labels).to(dev)
    T, Ds, Dt, V = w.T, w.Hs, w.Ht, w.V
    ws = torch.empty(flce.distill_workspace_bytes(T, Ds, Dt, V, chunk_rows), dtype=torch.uint8,
                     device=dev)
    kl = torch.empty(T, dtype=torch.float32, device=dev)
    mean = torch.empty((), dtype=torch.float32, device=dev)
    dh = torch.empty((T, Ds), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((V, Ds), dtype=torch.float32, device=dev)
    one = torch.ones((), dtype=torch.float32, device=dev)

    def step():
        flce.distill(sh, sw, th, tw, y, chunk_rows=chunk_rows, transform=xf, grad_mean=one,
                     grad_hidden=dh, grad_weight=dw, workspace=ws, kl=kl, mean=mean,
                     divergence=args.divergence, beta=args.beta)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    if args.divergence == "kl":
        flops = 4.0 * T * V * Dt + 8.0 * T * V * Ds
        passes = "2 lse passes, teacher and student block passes, dH, dW"
        loss = "mean KL(teacher || student)"
    else:  # one more teacher + student pass: the gradient needs each row's full sum first
        flops = 6.0 * T * V * Dt + 10.0 * T * V * Ds
        passes = ("2 lse passes, teacher and student statistics passes, teacher and student "
                  "gradient passes, dH, dW")
        loss = f"mean generalized JSD (beta {args.beta})"
    achieved = flops / (ms / 1e3)
    # per-kernel FLOPs per step: both log-sum-exp passes, the block passes of each head
    # (the JSD's gradient needs a second one of each), the student's dH and dW
    npass = 1 if args.divergence == "kl" else 2
    kernels, inst = kernel_breakdown(
        step, max(3, min(args.steps, 10)),
        {"fwd_lse": 2.0 * T * V * (Dt + Ds), "dst_teacher": npass * 2.0 * T * V * Dt,
         "dst_student": npass * 2.0 * T * V * Ds, "dst_dh": 2.0 * T * V * Ds,
         "dst_dw": 2.0 * T * V * Ds})
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    line = {
        "metric": "distillation fwd+bwd tokens/s (student and teacher LM heads)",
        "value": round(T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "student_hidden": Ds,
                   "teacher_hidden": Dt, "vocab": V, "chunk_rows": chunk_rows,
                   "masked_tokens": w.ignore_count, "loss": loss},
        "workspace_bytes": int(ws.numel()),
        "whole_call": {"passes": passes, "achieved": round(achieved / 1e12, 2),
                       "frac": round(achieved / PEAK_BF16, 4), "flops_per_step": flops},
        "roofline": {
            "kernel": dom, "bound": "mfma", "achieved": kernels[dom]["achieved"],
            "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": kernels[dom]["frac"],
            "traffic": None,
            "algorithmic_flops_per_launch": kernels[dom]["algorithmic_flops_per_launch"],
            "launches_per_step": kernels[dom]["launches_per_step"],
            "avg_launch_us": kernels[dom]["avg_launch_us"],
            "kernels": kernels, "instrumented": inst,
            "note": "the GEMM kernel with the most time per step, from the library's "
                    "per-launch events over instrumented steps after the timed ones",
        },
    }
    print(f"[bench] {args.workload}: inputs drawn in {t_gen:.1f} s; step {ms:.3f} ms",
          file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = distill_cpu_baseline(x, min(args.cpu_sample_tokens, T),
                                                    args.cpu_sample_vocab, args.divergence,
                                                    args.beta)
    print(json.dumps(line), flush=True)


# loss parameters of the policy workloads (GRPO: DeepSeekMath's beta and clip range)
POLICY_PARAMS = dict(grpo=dict(beta=0.04, eps_low=0.2, eps_high=0.2), dpo=dict(beta=0.1),
                     kto=dict(beta=0.1, desirable_weight=1.0, undesirable_weight=1.33))


def policy_main(args):
    """One step = one flce_{grpo,dpo,kto}_loss call with gradients: the fused log-prob
    forward, the loss kernels and the log-prob backward over the whole batch."""
    import numpy as np
    import torch

    from chunked_lm_head_amd import flce, synth

    w = synth.POLICY_WORKLOADS[args.workload]
    chunk_rows = args.chunk_rows or w.chunk_rows
    t_gen = time.perf_counter()
    x = synth.make_policy_inputs(w)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    h, W = bf16(x.hidden), bf16(x.weight)
    y = torch.from_numpy(x.labels).to(dev)
    T, D, V, B = w.T, w.H, w.V, w.n_seq
    prm = POLICY_PARAMS[args.loss]
    # side inputs near the policy's own log-probs, formed before the timed region
    lp, _, _ = flce.forward(h, W, y, chunk_rows=chunk_rows, mode="logprob")
    noise = {k: torch.from_numpy(getattr(x, k)).to(dev)
             for k in ("advantages", "old_noise", "ref_noise", "seq_noise")}
    mask = y != synth.IGNORE_INDEX
    pi = torch.where(mask, lp, 0.0).view(B, -1).double().sum(dim=1)
    ws = torch.empty(flce.policy_workspace_bytes(T, D, V, chunk_rows, B), dtype=torch.uint8,
                     device=dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    logp = torch.empty(T, dtype=torch.float32, device=dev)
    dh = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((V, D), dtype=torch.float32, device=dev)
    one = torch.ones((), dtype=torch.float32, device=dev)
    common = dict(chunk_rows=chunk_rows, grad_loss=one, grad_hidden=dh, grad_weight=dw,
                  workspace=ws, loss=loss, logp=logp)
    if args.loss == "grpo":
        old = (lp + 0.15 * noise["old_noise"]).float().contiguous()
        ref = (lp + 0.3 * noise["ref_noise"]).float().contiguous()

        def step():
            flce.grpo_loss(h, W, y, B, noise["advantages"], old_logp=old, ref_logp=ref,
                           **prm, **common)
    elif args.loss == "dpo":
        ref_seq = (pi + (1.5 / prm["beta"]) * noise["seq_noise"].double()).float().contiguous()

        def step():
            flce.dpo_loss(h, W, y, B, ref_seq, **prm, **common)
    else:
        ref_seq = (pi + (1.5 / prm["beta"]) * noise["seq_noise"].double()).float().contiguous()
        des = torch.from_numpy(x.desirable).to(dev)
        kl_ref = torch.tensor(0.05, dtype=torch.float32, device=dev)

        def step():
            flce.kto_loss(h, W, y, B, ref_seq, des, kl_ref=kl_ref, **prm, **common)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # prompt tokens carry no label and so no gradient: the backward skips their tiles, and
    # so does the log-prob forward (nothing needs their log-probs), the same tiles as the
    # recompute's
    bwd = backward_flops(x.labels != synth.IGNORE_INDEX,
                         flce.describe_plan(T, D, V, chunk_rows)["row_block"], V, D)
    gemm_flops = {"fwd_lse": bwd["bwd_grad"],
                  **{k: bwd[k] for k in ("bwd_grad", "bwd_dh", "bwd_dw")}}
    flops = sum(gemm_flops.values())
    achieved = flops / (ms / 1e3)
    kernels, inst = kernel_breakdown(step, max(3, min(args.steps, 10)), gemm_flops)
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    line = {
        "metric": f"{args.loss.upper()} loss fwd+bwd tokens/s (fused LM head, selective log-softmax)",
        "value": round(T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "loss": args.loss, "tokens": T, "hidden": D,
                   "vocab": V, "sequences": B, "seq_len": w.seq_len,
                   "prompt_tokens_per_sequence": w.prompt_len, "chunk_rows": chunk_rows,
                   "params": prm},
        "loss_value": round(float(loss.cpu()), 6),
        "workspace_bytes": int(ws.numel()),
        "whole_call": {"achieved": round(achieved / 1e12, 2),
                       "frac": round(achieved / PEAK_BF16, 4), "flops_per_step": flops,
                       "skipped_token_tiles": f"{bwd['skipped_token_tiles']} of "
                                              f"{bwd['token_tiles']}",
                       "note": "log-prob forward, loss kernels, recompute, dH, dW: FLOPs "
                               "executed (token tiles holding prompt tokens only are skipped "
                               "by the forward and the backward)"},
        "roofline": {
            "kernel": dom, "bound": "mfma", "achieved": kernels[dom]["achieved"],
            "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": kernels[dom]["frac"],
            "traffic": None,
            "algorithmic_flops_per_launch": kernels[dom]["algorithmic_flops_per_launch"],
            "launches_per_step": kernels[dom]["launches_per_step"],
            "avg_launch_us": kernels[dom]["avg_launch_us"],
            "kernels": kernels, "instrumented": inst,
            "note": "the GEMM kernel with the most time per step, from the library's "
                    "per-launch events over instrumented steps after the timed ones",
        },
    }
    print(f"[bench] {args.workload} {args.loss}: inputs drawn in {t_gen:.1f} s; step {ms:.3f} ms",
          file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = policy_cpu_baseline(x, args.loss, prm,
                                                   min(args.cpu_sample_tokens, T))
    print(json.dumps(line), flush=True)


def policy_cpu_baseline(x, loss: str, prm: dict, n_tokens: int) -> dict:
    """The oracle, untouched, on the first n_tokens tokens against the whole vocabulary:
    log-probs, the loss (the sample as one sequence, or for DPO its halves as one pair;
    on-policy ratios, reference = policy) and the log-prob backward."""
    import numpy as np

    from oracle import policy_oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    h, wt, y = x.hidden[:n_tokens], x.weight, x.labels[:n_tokens]
    t0 = time.perf_counter()
    lp = policy_oracle.logp(h, wt, y)
    if loss == "grpo":
        r = policy_oracle.grpo_from_logp(lp, y, 1, x.advantages[:1], ref_logp=lp, **prm)
    elif loss == "dpo":  # the two halves of the sample as one chosen / rejected pair
        r = policy_oracle.dpo_from_logp(lp, y, 2, np.zeros(2), **prm)
    else:
        r = policy_oracle.kto_from_logp(lp, y, 1, np.zeros(1), x.desirable[:1], **prm)
    policy_oracle.grads(h, wt, y, r.dlogp)
    dt = time.perf_counter() - t0
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"first {n_tokens} tokens x all {wt.shape[0]} vocabulary rows, float64 "
                      f"numpy log-probs + {loss.upper()} loss + backward in {dt:.1f} s"}


def distill_cpu_baseline(x, n_tokens: int, n_vocab: int, divergence: str = "kl",
                         beta: float = 0.5) -> dict:
    """The distillation oracle, untouched, on the first n_tokens tokens against the first
    n_vocab vocabulary rows of both heads; the rate is scaled by n_vocab / V."""
    from oracle import distill_oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    V = x.s_weight.shape[0]
    n_vocab = min(n_vocab, V)
    args = (x.s_hidden[:n_tokens], x.s_weight[:n_vocab], x.t_hidden[:n_tokens],
            x.t_weight[:n_vocab], x.labels[:n_tokens])
    t0 = time.perf_counter()
    distill_oracle.forward(*args, divergence=divergence, beta=beta)
    distill_oracle.backward(*args, grad_mean=1.0, divergence=divergence, beta=beta)
    dt = time.perf_counter() - t0
    return {"value": round(n_tokens / dt * n_vocab / V, 3), "unit": "tokens/s",
            "cores": int(cores), "kind": "oracle",
            "sample": f"first {n_tokens} tokens x first {n_vocab} of {V} vocabulary rows of "
                      f"both heads, float64 numpy forward + backward in {dt:.1f} s; rate scaled "
                      f"by {n_vocab}/{V}"}


class PowerSampler:
    """Samples socket power and the GFX clocks with `amd-smi metric -p -c` in a thread
    (a read-only query, about twice a second) while the timed steps run."""

    def __init__(self):
        import threading
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import re
        import subprocess
        while not self._stop.is_set():
            try:
                out = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True,
                                     text=True, timeout=5).stdout
            except Exception:  # pragma: no cover - tool missing or slow
                return
            w = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", out)
            clks = [float(c) for c in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", out)]
            if w:
                self.samples.append((float(w.group(1)), clks))
            self._stop.wait(0.4)

    def start(self):
        self._thread.start()

    def stop(self) -> dict:
        self._stop.set()
        self._thread.join(timeout=10)
        s = self.samples[1:] or self.samples  # the first sample may precede the load
        if not s:
            return {"samples": 0}
        watts = [w for w, _ in s]
        clks = [c for _, cs in s for c in cs]
        return {"samples": len(s), "socket_w_mean": round(sum(watts) / len(watts), 1),
                "socket_w_max": max(watts), "cap_w": 1400.0,
                "gfx_clk_mhz_mean": round(sum(clks) / len(clks), 0) if clks else None}


def gemm_ceiling(w) -> None:
    """Vendor bf16 GEMMs (plain 2-D torch.mm, fp32 accumulate, bf16 out) at the logit
    shape T x V x D and at the backward block shapes, as a practical ceiling."""
    import torch

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)

    def rnd(*shape):
        return torch.randn(*shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)

    def timeit(fn, flops, reps=5):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        return ms, flops / (ms / 1e3) / 1e12

    T, D, V = w.T, w.H, w.V
    res = {}
    h, W = rnd(T, D), rnd(V, D)
    z = torch.empty(T, V, dtype=torch.bfloat16, device=dev)
    res["logits_T_V_D"] = timeit(lambda: torch.mm(h, W.t(), out=z), 2.0 * T * V * D)
    del z
    R, Vc = min(T, 8192), 8192
    G = rnd(R, Vc)
    Wc = W[:Vc].contiguous()
    hb = h[:R].contiguous()
    res["dH_R_D_Vc"] = timeit(lambda: torch.mm(G, Wc), 2.0 * R * Vc * D)
    res["dW_Vc_D_R"] = timeit(lambda: torch.mm(G.t(), hb), 2.0 * R * Vc * D)
    out = {k: {"ms": round(v[0], 3), "TFLOP/s": round(v[1], 1),
               "frac_of_2.5PF": round(v[1] / (PEAK_BF16 / 1e12), 4)} for k, v in res.items()}
    print(json.dumps({"gemm_ceiling": out, "workload": w.name}), flush=True)


def _kernel_sha() -> str:
    import hashlib

    hsh = hashlib.sha256()
    for f in ("flce_tile.hpp", "flce_kernels.hpp", "flce_api.hip"):
        with open(os.path.join(ROOT, "chunked_lm_head_amd", "csrc", f), "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()[:16]


if __name__ == "__main__":
    main()
