"""The C-ABI library on the host: it loads, exports what include/flce.h declares, and
rejects bad arguments before touching a GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def flce():
    from chunked_lm_head_amd import flce as m
    return m


def _declared():
    src = open(os.path.join(ROOT, "include", "flce.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(flce):
    names = _declared()
    assert set(names) == set(flce.EXPORTS), names
    for n in names:
        assert hasattr(flce.lib, n), n


def test_status_strings(flce):
    for s in range(6):
        assert flce.lib.flce_status_string(s)
    assert b"unknown" in flce.lib.flce_status_string(99)


def test_shape_checks(flce):
    ws = flce.lib.flce_workspace_bytes
    assert ws(-1, 64, 100, 16) == 0
    assert ws(10, 0, 100, 16) == 0
    assert ws(10, 64, 0, 16) == 0
    assert ws(10, 64, 100, 0) == 0
    assert ws(10, 60, 100, 16) == 0        # D not a multiple of 8
    assert ws(0, 64, 100, 16) > 0          # empty batch is valid
    assert ws(67, 128, 1000, 16) > 0


def _fwd(flce, **over):
    args = dict(hidden=16, weight=16, labels=8, T=4, D=64, V=100, ign=-100, cr=16, mode=0,
                xf=None, out=4, lse=4, mean=0, ws=16, wsb=1 << 30, stream=0)
    args.update(over)
    return flce.lib.flce_forward(args["hidden"], args["weight"], args["labels"], args["T"],
                                 args["D"], args["V"], args["ign"], args["cr"], args["mode"],
                                 args["xf"], args["out"], args["lse"], args["mean"] or None, args["ws"],
                                 args["wsb"], args["stream"] or None)


def test_forward_rejects_before_launch(flce):
    assert _fwd(flce, T=-3) == 2
    assert _fwd(flce, D=12) == 4
    assert _fwd(flce, mode=7) == 1
    assert _fwd(flce, hidden=0) == 1
    assert _fwd(flce, hidden=8) == 1                 # misaligned
    assert _fwd(flce, wsb=16) == 3                   # workspace too small
    assert b"workspace" in flce.lib.flce_last_error()


def test_forward_noalloc_rejects_before_launch(flce):
    f = flce.lib.flce_forward_noalloc

    def call(**over):
        a = dict(hidden=16, weight=16, labels=8, T=4, D=64, V=100, ign=-100, cr=16, mode=0,
                 xf=None, out=4, lse=4, mean=None, stream=None)
        a.update(over)
        return f(a["hidden"], a["weight"], a["labels"], a["T"], a["D"], a["V"], a["ign"],
                 a["cr"], a["mode"], a["xf"], a["out"], a["lse"], a["mean"], a["stream"])

    assert call(T=-3) == 2
    assert call(D=12) == 4
    assert call(mode=7) == 1
    assert call(hidden=None) == 1
    assert call(hidden=8) == 1                      # misaligned
    # the forward's partial results outgrow the fixed 16 MiB array past ~1.39M tokens
    assert call(T=1_400_000, D=4096, V=151936) == 3
    assert b"scratch" in flce.lib.flce_last_error()


def test_backward_rejects_before_launch(flce):
    b = flce.lib.flce_backward
    # neither grad given
    assert b(16, 16, 8, 4, 4, 64, 100, -100, 16, 0, None, None, None, 16, 16, 0, 16, 1 << 30, None) == 1
    # both given
    assert b(16, 16, 8, 4, 4, 64, 100, -100, 16, 0, None, 4, 4, 16, 16, 0, 16, 1 << 30, None) == 1
    # neither gradient output given (either alone is allowed: the other is skipped)
    assert b(16, 16, 8, 4, 4, 64, 100, -100, 16, 0, None, 4, None, None, None, 0, 16, 1 << 30, None) == 1
    assert b"both NULL" in flce.lib.flce_last_error()
    # tiny workspace
    assert b(16, 16, 8, 4, 4, 64, 100, -100, 16, 0, None, 4, None, 16, 16, 0, 16, 8, None) == 3


def test_timing_rejects_before_any_device_call(flce):
    lib = flce.lib
    assert lib.flce_timing_begin(0) == 1
    assert lib.flce_timing_begin(1 << 21) == 1
    assert b"capacity" in lib.flce_last_error()
    ids, ms = (ctypes.c_int32 * 4)(), (ctypes.c_float * 4)()
    n = ctypes.c_int32()
    assert lib.flce_timing_end(ids, ms, 4, ctypes.byref(n), None) == 1     # timing is off
    assert b"not on" in lib.flce_last_error()
    assert lib.flce_timing_end(None, ms, 4, ctypes.byref(n), None) == 1
    names = [lib.flce_kernel_name(i).decode() for i in range(1, 22)]
    assert len(set(names)) == 21 and "?" not in names
    assert lib.flce_kernel_name(0) == b"?" and lib.flce_kernel_name(22) == b"?"
    assert names[5:8] == ["bwd_grad", "bwd_dh", "bwd_dw"]


BAD_TRANSFORMS = [
    (-1.0, 0.0, 0.0, 1.0),            # negative multiply
    (0.0, -2.0, 0.0, 1.0),            # negative divide
    (0.0, 0.0, -30.0, 1.0),           # negative softcap
    (0.0, 0.0, 0.0, 0.0),             # zero temperature
    (0.0, 0.0, 0.0, -1.0),            # negative temperature
    (float("nan"), 0.0, 0.0, 1.0),
    (0.0, 0.0, float("inf"), 1.0),
    (0.0, 0.0, 0.0, float("inf")),
    (1e30, 1e-30, 0.0, 1.0),          # combined scale overflows fp32
    (0.0, 0.0, 1e-39, 1.0),           # 1 / softcap overflows fp32
]


@pytest.mark.parametrize("vals", BAD_TRANSFORMS)
def test_invalid_logit_transform_rejected(flce, vals):
    xf = ctypes.byref(flce.LogitTransform(*vals))
    assert _fwd(flce, xf=xf) == 1
    assert b"transform" in flce.lib.flce_last_error()
    b = flce.lib.flce_backward
    assert b(16, 16, 8, 4, 4, 64, 100, -100, 16, 0, xf, 4, None, 16, 16, 0, 16, 1 << 30,
             None) == 1


def test_identity_transform_is_none(flce):
    assert flce.make_transform() is None
    assert flce.make_transform(temperature=0.7) is not None


def test_workspace_bound_independent_of_tokens_times_vocab(flce):
    """Workspace: at most one chunk of fp32 logits (chunk_rows*V*4) for the bf16 gradient
    block, plus terms linear in T and in D; the long-context shape needs about what the
    16k-token shape needs although T*V is 8x larger."""
    D, V, cr = 4096, 151936, 256
    a = flce.describe_plan(16384, D, V, cr)
    b = flce.describe_plan(131072, D, V, cr)
    assert a["grad_tile_bytes"] <= cr * V * 4 and b["grad_tile_bytes"] <= cr * V * 4
    wa, wb = flce.workspace_bytes(16384, D, V, cr), flce.workspace_bytes(131072, D, V, cr)
    assert wb - wa <= 64 * (131072 - 16384)          # O(T) growth only
    assert wb < 0.02 * 131072 * V * 4                 # far below the full fp32 logits
    for T, D, V, cr in [(67, 128, 1000, 16), (256, 2048, 248320, 256), (32768, 4096, 128000, 256),
                        (8500, 64, 700, 256), (300, 256, 5000, 1)]:
        p = flce.describe_plan(T, D, V, cr)
        assert p["grad_tile_bytes"] <= max(cr * V * 4, 256 * 256 * 2)
        assert p["row_block"] % 256 == 0 and p["vocab_chunk"] % 256 == 0
        assert p["row_block"] * p["row_blocks"] >= T
        assert p["vocab_chunk"] * p["vocab_chunks"] >= V
        assert (p["vocab_chunks"] - 1) * p["vocab_chunk"] < V
        assert (p["row_blocks"] - 1) * p["row_block"] < T
        assert p["fwd_splits"] <= p["vocab_tiles"]


def test_plan_at_the_workload_shapes(flce):
    p = flce.describe_plan(16384, 4096, 151936, 256)
    assert p["token_tiles"] == 64 and p["vocab_tiles"] == 594
    assert p["token_tiles"] * p["fwd_splits"] >= 1024
    p = flce.describe_plan(256, 2048, 248320, 256)
    assert p["vocab_chunks"] == 1 and p["row_blocks"] == 1
    # the full-size goldens sample tokens and dW rows on both sides of these row-block and
    # vocabulary-chunk edges, so the plans at those shapes are fixed here
    for T, V, rb, vc in [(16384, 151936, 8192, 8192), (32768, 128000, 8192, 7936),
                         (131072, 151936, 8192, 8192)]:
        p = flce.describe_plan(T, 4096, V, 256)
        assert (p["row_block"], p["vocab_chunk"], p["dh_splits"]) == (rb, vc, 1), (T, V, p)
    p = flce.describe_plan(256, 2048, 248320, 256)
    assert (p["row_block"], p["vocab_chunk"], p["dh_splits"]) == (256, 248320, 32), p


def _dst(flce, **over):
    a = dict(sh=16, sw=16, Ds=64, th=16, tw=16, Dt=96, labels=None, ign=-100, T=4, V=100, cr=16,
             xf=None, kl=4, mean=None, gout=None, gmean=None, gh=None, gw=None, acc=0, ws=16,
             wsb=1 << 30, stream=None)
    a.update(over)
    return flce.lib.flce_distill(a["sh"], a["sw"], a["Ds"], a["th"], a["tw"], a["Dt"],
                                 a["labels"], a["ign"], a["T"], a["V"], a["cr"], a["xf"],
                                 a["kl"], a["mean"], a["gout"], a["gmean"], a["gh"], a["gw"],
                                 a["acc"], a["ws"], a["wsb"], a["stream"])


def test_distill_rejects_before_launch(flce):
    assert _dst(flce, T=-1) == 2
    assert _dst(flce, Ds=60) == 4                    # student hidden not a multiple of 8
    assert _dst(flce, Dt=12) == 4                    # teacher hidden not a multiple of 8
    assert _dst(flce, gout=4, gmean=4, gh=16, gw=16) == 1   # both upstream grads
    assert _dst(flce, gmean=4) == 1                  # gradient with neither output
    assert b"both NULL" in flce.lib.flce_last_error()
    assert _dst(flce, th=0) == 1
    assert _dst(flce, tw=8) == 1                     # misaligned
    assert _dst(flce, wsb=16) == 3
    bad = ctypes.byref(flce.LogitTransform(0.0, 0.0, 0.0, 0.0))
    assert _dst(flce, xf=bad) == 1


def test_distill_workspace_bound(flce):
    wb = flce.lib.flce_distill_workspace_bytes
    assert wb(10, 60, 64, 100, 16) == 0
    assert wb(10, 64, 0, 100, 16) == 0
    assert wb(0, 64, 64, 100, 16) > 0
    # the p_t block (fp32, G written over it) within one chunk of fp32 logits, plus terms
    # linear in T and D
    for T, Ds, Dt, V, cr in [(16384, 4096, 5120, 151936, 256), (131072, 4096, 4096, 151936, 256),
                             (4096, 2048, 4096, 248320, 64)]:
        n = wb(T, Ds, Dt, V, cr)
        linear = 64 * T * 4 + 256 * 4 * 8192 * 4 + 8192 * Ds * 4 * 2 + (32 << 20)
        assert n <= cr * V * 4 + linear, (T, V, n)
        assert n < T * V * 4 / 10


def _pol(flce, kind="grpo", **over):
    a = dict(h=16, w=16, labels=16, ign=-100, T=8, D=64, V=100, cr=16, xf=None, n_seq=2,
             adv=16, old=None, ref=None, refseq=16, des=16, klref=None,
             prm=ctypes.byref(flce.PolicyParams(0.1, 0.2, 0.2, 1.0, 1.0)), loss=4, logp=None,
             gl=None, gh=None, gw=None, acc=0, ws=16, wsb=1 << 30, stream=None)
    a.update(over)
    head = (a["h"], a["w"], a["labels"], a["ign"], a["T"], a["D"], a["V"], a["cr"], a["xf"],
            a["n_seq"])
    tail = (a["prm"], a["loss"], a["logp"], a["gl"], a["gh"], a["gw"], a["acc"], a["ws"],
            a["wsb"], a["stream"])
    if kind == "grpo":
        return flce.lib.flce_grpo_loss(*head, a["adv"], a["old"], a["ref"], *tail)
    if kind == "dpo":
        return flce.lib.flce_dpo_loss(*head, a["refseq"], *tail)
    return flce.lib.flce_kto_loss(*head, a["refseq"], a["des"], a["klref"], *tail)


def _prm(flce, *v):
    return ctypes.byref(flce.PolicyParams(*v))


@pytest.mark.parametrize("kind", ["grpo", "dpo", "kto"])
def test_policy_rejects_before_launch(flce, kind):
    assert _pol(flce, kind, n_seq=3) == 2            # n_seq does not divide T
    assert _pol(flce, kind, n_seq=0) == 2
    assert _pol(flce, kind, T=-1) == 2
    assert _pol(flce, kind, D=60) == 4
    assert _pol(flce, kind, prm=None) == 1
    assert _pol(flce, kind, loss=None) == 1
    assert _pol(flce, kind, gl=4) == 1               # gradient with neither output
    assert b"both NULL" in flce.lib.flce_last_error()
    assert _pol(flce, kind, h=None) == 1
    assert _pol(flce, kind, h=8) == 1                # misaligned
    assert _pol(flce, kind, wsb=16) == 3
    bad = ctypes.byref(flce.LogitTransform(0.0, 0.0, 0.0, -1.0))
    assert _pol(flce, kind, xf=bad) == 1


def test_policy_parameter_checks(flce):
    assert _pol(flce, "grpo", adv=None) == 1
    assert _pol(flce, "grpo", prm=_prm(flce, -0.1, 0.2, 0.2, 0, 0)) == 1   # beta < 0
    assert _pol(flce, "grpo", prm=_prm(flce, 0.0, 1.0, 0.2, 0, 0)) == 1    # eps_low >= 1
    assert _pol(flce, "grpo", prm=_prm(flce, 0.0, 0.2, -0.5, 0, 0)) == 1   # eps_high < 0
    assert _pol(flce, "grpo", prm=_prm(flce, float("nan"), 0.2, 0.2, 0, 0)) == 1
    assert _pol(flce, "dpo", refseq=None) == 1
    assert _pol(flce, "dpo", T=6, n_seq=3) == 2     # DPO pairs need an even count
    assert _pol(flce, "dpo", prm=_prm(flce, 0.0, 0, 0, 0, 0)) == 1         # beta must be > 0
    assert _pol(flce, "kto", des=None) == 1
    assert _pol(flce, "kto", prm=_prm(flce, 0.1, 0, 0, -1.0, 1.0)) == 1    # weight < 0
    assert _pol(flce, "kto", prm=_prm(flce, 0.1, 0, 0, 1.0, float("inf"))) == 1


def test_policy_workspace_bytes(flce):
    pb = flce.lib.flce_policy_workspace_bytes
    assert pb(8, 64, 100, 16, 3) == 0
    assert pb(8, 64, 100, 16, 0) == 0
    assert pb(8, 60, 100, 16, 2) == 0
    for T, D, V, cr, n in [(32768, 4096, 128000, 256, 4), (8, 64, 100, 16, 8), (0, 64, 100, 16, 1)]:
        base = flce.lib.flce_workspace_bytes(T, D, V, cr)
        got = pb(T, D, V, cr, n)
        assert base + 12 * T + 16 * n <= got <= base + 12 * T + 16 * n + 7 * 256, (T, got, base)


def test_distill_jsd_rejects_before_launch(flce):
    def call(beta, **over):
        a = dict(sh=16, sw=16, Ds=64, th=16, tw=16, Dt=96, labels=None, ign=-100, T=4, V=100,
                 cr=16, xf=None, kl=4, mean=None, gout=None, gmean=None, gh=None, gw=None, acc=0,
                 ws=16, wsb=1 << 30, stream=None)
        a.update(over)
        return flce.lib.flce_distill_jsd(a["sh"], a["sw"], a["Ds"], a["th"], a["tw"], a["Dt"],
                                         a["labels"], a["ign"], a["T"], a["V"], a["cr"], a["xf"],
                                         beta, a["kl"], a["mean"], a["gout"], a["gmean"], a["gh"],
                                         a["gw"], a["acc"], a["ws"], a["wsb"], a["stream"])

    for beta in (0.0, 1.0, -0.5, 1.5, float("nan")):
        assert call(beta) == 1, beta                  # the weight must lie in (0, 1)
    assert call(0.5, T=-1) == 2
    assert call(0.5, Ds=60) == 4
    assert call(0.5, gmean=4) == 1                   # gradient with neither output
    assert call(0.5, tw=8) == 1                      # misaligned
    assert call(0.5, wsb=16) == 3
