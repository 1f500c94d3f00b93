"""flce_forward_noalloc (the library's fixed scratch array, no workspace) gives the same
outputs as flce_forward with a caller workspace, on two calls in a row, the second with a
smaller input; nothing is allocated by the call."""
import numpy as np
import pytest
import torch

from chunked_lm_head_amd import synth
from oracle import flce_oracle as o

import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case(name, T, D, V, seed, mode):
    w = synth.custom(name, T=T, H=D, V=V, chunk_rows=64, ignore_frac=0.05, mode=mode, seed=seed)
    return w, synth.make_inputs(w)


@pytest.mark.parametrize("first,second", [((4100, 256, 3000), (300, 128, 1000))])
def test_noalloc_forward_matches_the_workspace_forward(first, second):
    from chunked_lm_head_amd import flce

    dev = gu.device()
    for k, (T, D, V) in enumerate((first, second)):
        mode = ("nll", "logprob")[k]
        w, x = _case(f"noalloc{k}", T, D, V, 91 + k, mode)
        print(f"case noalloc call {k}: T={T} D={D} V={V} {mode}", flush=True)
        h, W = gu.bf16_tensor(x.hidden, dev), gu.bf16_tensor(x.weight, dev)
        y = torch.from_numpy(x.labels).to(dev)
        tr = dict(logit_softcapping=4.0, temperature=0.8) if k else {}
        out, lse, mean = flce.forward(h, W, y, chunk_rows=w.chunk_rows, mode=mode,
                                      transform=tr)
        out2 = torch.empty(T, dtype=torch.float32, device=dev)
        lse2 = torch.empty(T, dtype=torch.float32, device=dev)
        mean2 = torch.empty((), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(dev)
        flce.forward_noalloc(h, W, y, chunk_rows=w.chunk_rows, mode=mode, transform=tr,
                             out=out2, lse=lse2, mean=mean2)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated(dev) == before
        # same kernels and plan: the same bits
        assert torch.equal(out2, out) and torch.equal(lse2, lse) and torch.equal(mean2, mean)
        # and within the tolerance of the oracle
        f = o.forward(x.hidden, x.weight, x.labels, synth.IGNORE_INDEX, mode,
                      transform=o.LogitTransform(softcap=4.0, temperature=0.8) if k else None)
        assert gu.max_abs(out2.cpu().numpy(), f.out) <= gu.OUT_TOL
        assert gu.max_abs(lse2.cpu().numpy(), f.lse) <= gu.OUT_TOL
        assert abs(float(mean2.cpu()) - f.mean) <= gu.OUT_TOL


def test_noalloc_forward_refuses_a_batch_beyond_its_array():
    from chunked_lm_head_amd import flce

    dev = gu.device()
    T, D, V = 1_400_000, 8, 300
    h = torch.zeros((T, D), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((V, D), dtype=torch.bfloat16, device=dev)
    y = torch.zeros(T, dtype=torch.int64, device=dev)
    out = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    with pytest.raises(flce.FlceError, match="scratch"):
        flce.forward_noalloc(h, W, y, out=out, lse=lse)
