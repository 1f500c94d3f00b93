"""Helpers shared by the GPU tests: run the HIP path through the C ABI and compare."""
from __future__ import annotations

import numpy as np
import torch

from chunked_lm_head_amd import synth

OUT_TOL = 2e-3     # per-token |loss or log-prob error|
GRAD_TOL = 1e-2    # relative Frobenius error of dH and dW


def device():
    return torch.device("cuda:0")


def bf16_tensor(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def binding_transform(tr) -> dict:
    """Keyword arguments of the binding for a transform given as
    (multiply, divide, softcap, temperature) or an object with those fields."""
    if tr is None:
        return {}
    if not isinstance(tr, (tuple, list, np.ndarray)):
        tr = (tr.scale_multiply, tr.scale_divide, tr.softcap, tr.temperature)
    m, d, c, t = (float(v) for v in tr)
    return dict(logit_scale_multiply=m, logit_scale_divide=d, logit_softcapping=c,
                temperature=t)


def run(x: synth.Inputs, *, chunk_rows=None, mode=None, grad_out=None, grad_mean=1.0,
        labels=None, weight_bits=None, accumulate_into=None, transform=None):
    """Forward + backward through the library; returns numpy arrays."""
    from chunked_lm_head_amd import flce

    w = x.workload
    dev = device()
    chunk_rows = w.chunk_rows if chunk_rows is None else chunk_rows
    mode = w.mode if mode is None else mode
    h = bf16_tensor(x.hidden, dev)
    W = bf16_tensor(x.weight if weight_bits is None else weight_bits, dev)
    y = torch.from_numpy(x.labels if labels is None else labels).to(dev)
    xf = binding_transform(transform)
    out, lse, mean = flce.forward(h, W, y, chunk_rows=chunk_rows, mode=mode, transform=xf)
    g = x.grad_out if grad_out is None else grad_out
    kw = {}
    if g is not None:
        kw["grad_out"] = torch.from_numpy(np.asarray(g, dtype=np.float32)).to(dev)
    else:
        kw["grad_mean"] = torch.tensor(float(grad_mean), dtype=torch.float32, device=dev)
    gw = None
    if accumulate_into is not None:
        gw = torch.from_numpy(accumulate_into.astype(np.float32)).to(dev)
    dh, dw = flce.backward(h, W, y, lse, chunk_rows=chunk_rows, mode=mode, transform=xf,
                           grad_weight=gw,
                           accumulate=accumulate_into is not None, **kw)
    torch.cuda.synchronize()
    return dict(out=out.cpu().numpy(), lse=lse.cpu().numpy(), mean=float(mean.cpu()),
                dh=dh.float().cpu().numpy(), dw=dw.cpu().numpy())


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    d = float(np.linalg.norm(np.asarray(a, dtype=np.float64) - b))
    return d / nb if nb > 0 else d


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - b))) if np.size(b) else 0.0
