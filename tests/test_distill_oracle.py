"""The distillation oracle against its pins, and mutants of it that some pin must catch."""
import os
import sys
import types
import warnings

import pytest

import distill_pins as pins
from oracle import distill_oracle as d

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "distill_oracle.py")


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_distill_pin(check):
    check(d)


MUTANTS = {
    "reverse_kl": ("kl[r0:r1] = (np.exp(log_pt) * (log_pt - log_ps)).sum(axis=1)",
                   "kl[r0:r1] = (np.exp(log_ps) * (log_ps - log_pt)).sum(axis=1)"),
    "cross_entropy_not_kl": ("kl[r0:r1] = (np.exp(log_pt) * (log_pt - log_ps)).sum(axis=1)",
                             "kl[r0:r1] = (np.exp(log_pt) * (-log_ps)).sum(axis=1)"),
    "grad_sign": ("g = (np.exp(_log_softmax(zs)) - np.exp(_log_softmax(zt))) * c[:, None]",
                  "g = (np.exp(_log_softmax(zt)) - np.exp(_log_softmax(zs))) * c[:, None]"),
    "teacher_untransformed": ("        zt, _ = _rows(ht, wt, transform, r0, r1)\n        lse_s",
                              "        zt, _ = _rows(ht, wt, None, r0, r1)\n        lse_s"),
    "mean_over_all_tokens": ("mean = float(kl[valid].sum() / n_valid) if n_valid else 0.0",
                             "mean = float(kl.sum() / T)"),
    "masked_tokens_get_grad": ("    return np.where(valid, g, 0.0)", "    return g"),
    "no_chain_rule": ("return g if dzs is None else g * dzs", "return g"),
    "weight_rows_no_teacher": ("g = np.exp(log_ps) - np.exp(log_pt)", "g = np.exp(log_ps)"),
    "lse_swapped": ("        log_pt = zt - lse_t[r0:r1, None]", "        log_pt = zt - lse_s[r0:r1, None]"),
    "jsd_mixture_weights_swapped": ("    m = beta * pt + (1.0 - beta) * ps",
                                    "    m = beta * ps + (1.0 - beta) * pt"),
    "jsd_teacher_term_weight": ("    return (beta * _xlogy_ratio(pt, log_pt, log_m)",
                                "    return ((1.0 - beta) * _xlogy_ratio(pt, log_pt, log_m)"),
    "jsd_grad_without_row_sum": ("g = ps * (gv - gbar) * c[:, None]", "g = ps * gv * c[:, None]"),
    "jsd_grad_weight": ("        gv = (1.0 - beta) * (log_ps - log_m)\n",
                        "        gv = beta * (log_ps - log_m)\n"),
    # row-blocked loops
    "block_scale_offset_dropped": ("g = grad_logits(zs, zt, c[r0:r1], dzs, divergence, beta)",
                                   "g = grad_logits(zs, zt, c[:r1 - r0], dzs, divergence, beta)"),
    "block_lse_offset_dropped": ("        lse_t[r0:r1] = fo.logsumexp_rows(zt)\n",
                                 "        lse_t[:r1 - r0] = fo.logsumexp_rows(zt)\n"),
    "block_gbar_offset_dropped": ("out[r0:r1] = (ps * gv).sum(axis=1)",
                                  "out[:r1 - r0] = (ps * gv).sum(axis=1)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not found once: {old!r}"
    modname = f"distill_oracle_mutant_{name}"
    mod = types.ModuleType(modname)
    sys.modules[modname] = mod          # dataclasses look the module up by name
    try:
        exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    finally:
        del sys.modules[modname]
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_distill_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    for check in pins.ALL_CHECKS:
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            try:
                check(mod)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"
