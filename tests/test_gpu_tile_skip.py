"""Token tiles without any gradient (a per-token upstream gradient that is zero on whole
256-token tiles, as on the prompt tokens of a policy loss) are left out of the backward
GEMMs: the tiles with a gradient are listed on the device and packed into the leading row
blocks, the recompute, dH and dW of each row block run over the tiles it holds, and the
left-out tiles' dH rows are written as zeros.  The results must match the oracle as
everywhere else, and the left-out tokens' dH rows must be exact zeros."""
import numpy as np
import pytest
import torch

from chunked_lm_head_amd import synth
from oracle import flce_oracle as o

import gpu_util as gu

pytestmark = pytest.mark.gpu

IGN = synth.IGNORE_INDEX


def _zero_tiles(T, tiles):
    """Upstream gradient ~N(0, 1) with the given 256-token tiles zeroed."""
    g = np.random.default_rng(91).standard_normal(T).astype(np.float32)
    for t in tiles:
        g[t * 256:(t + 1) * 256] = 0.0
    return g


# name, T, D, V, chunk_rows, zero tiles, mode: one row block with holes at the start, in
# the middle and at the ragged end; many one-tile row blocks (chunk_rows 16), of which the
# trailing ones end up empty once the active tiles are packed; all tiles but one
CASES = [
    ("holes_one_block", 2600, 264, 3100, 200, (0, 1, 5, 10), "logprob"),
    ("holes_nll", 2600, 264, 3100, 200, (2, 3, 4), "nll"),
    ("zero_row_blocks", 2100, 128, 3100, 16, (0, 3, 4, 8), "logprob"),
    ("all_but_one", 1500, 136, 2000, 200, (0, 1, 2, 4, 5), "nll"),
    # a last packed row block of one or two tiles, whose dH spreads its K range over many
    # more splits than planned (stacked in the same partial-sum buffer), over several
    # vocabulary chunks; the second with the batch's ragged last tile in that block
    ("small_packed_block", 4096, 264, 3100, 256, tuple(range(9, 16)), "logprob"),
    ("small_packed_ragged", 6000, 520, 3100, 1024, tuple(range(10)), "nll"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_tiles_without_gradient(case):
    from chunked_lm_head_amd import flce

    name, T, D, V, cr, tiles, mode = case
    w = synth.custom(name, T=T, H=D, V=V, chunk_rows=cr, ignore_frac=0.03, mode=mode, seed=92)
    x = synth.make_inputs(w)
    g = _zero_tiles(T, tiles)
    plan = flce.describe_plan(T, D, V, cr)
    print(f"case {name}: row blocks {plan['row_blocks']} of {plan['row_block']}, chunks "
          f"{plan['vocab_chunks']}, zero tiles {tiles}", flush=True)
    dev = gu.device()
    h, W = gu.bf16_tensor(x.hidden, dev), gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    _, lse, _ = flce.forward(h, W, y, chunk_rows=cr, mode=mode)
    dh, dw = flce.backward(h, W, y, lse, grad_out=torch.from_numpy(g).to(dev), chunk_rows=cr,
                           mode=mode)
    torch.cuda.synchronize()
    rdh, rdw = o.backward(x.hidden, x.weight, x.labels, IGN, mode, grad_out=g)
    dhg, dwg = dh.float().cpu().numpy(), dw.cpu().numpy()
    e_dh, e_dw = gu.rel_fro(dhg, rdh), gu.rel_fro(dwg, rdw)
    print(f"  dH rel {e_dh:.2e}  dW rel {e_dw:.2e}", flush=True)
    assert e_dh <= gu.GRAD_TOL and e_dw <= gu.GRAD_TOL, (e_dh, e_dw)
    zero_rows = np.concatenate([np.arange(t * 256, min(T, (t + 1) * 256)) for t in tiles])
    assert not np.any(dhg[zero_rows]), "skipped tokens must have exactly zero dH rows"
    # the same call twice gives the same bits (the skip decisions are made on the device)
    dh2, dw2 = flce.backward(h, W, y, lse, grad_out=torch.from_numpy(g).to(dev), chunk_rows=cr,
                             mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(dh, dh2) and torch.equal(dw, dw2)


def test_no_gradient_at_all_gives_zero_gradients():
    from chunked_lm_head_amd import flce

    w = synth.custom("no_grad", T=700, H=128, V=900, chunk_rows=64, ignore_frac=0.0, seed=93)
    x = synth.make_inputs(w)
    dev = gu.device()
    h, W = gu.bf16_tensor(x.hidden, dev), gu.bf16_tensor(x.weight, dev)
    y = torch.from_numpy(x.labels).to(dev)
    _, lse, _ = flce.forward(h, W, y, chunk_rows=w.chunk_rows)
    zero = torch.zeros(w.T, dtype=torch.float32, device=dev)
    dw = torch.full((w.V, w.H), 7.0, dtype=torch.float32, device=dev)
    dh, dw = flce.backward(h, W, y, lse, grad_out=zero, chunk_rows=w.chunk_rows,
                           grad_weight=dw)
    torch.cuda.synchronize()
    assert not torch.any(dh.float()) and not torch.any(dw)
    # accumulating zero gradients leaves grad_weight as it was
    dw.fill_(3.0)
    _, dw = flce.backward(h, W, y, lse, grad_out=zero, chunk_rows=w.chunk_rows, grad_weight=dw,
                          accumulate=True)
    torch.cuda.synchronize()
    assert bool(torch.all(dw == 3.0))
