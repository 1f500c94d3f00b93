"""The policy-loss oracle against its pins, and mutants of it that some pin must catch."""
import os
import sys
import types
import warnings

import pytest

import policy_pins as pins
from oracle import policy_oracle as p

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "policy_oracle.py")


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_policy_pin(check):
    check(p)


MUTANTS = {
    "clip_upper_uses_eps_low": ("np.clip(r, 1.0 - eps_low, 1.0 + eps_high)",
                                "np.clip(r, 1.0 - eps_low, 1.0 + eps_low)"),
    "surrogate_max": ("s = np.minimum(unclipped, clipped)", "s = np.maximum(unclipped, clipped)"),
    "clipped_branch_keeps_grad": ("ds = np.where(unclipped <= clipped, r * A, 0.0)",
                                  "ds = r * A"),
    "kl_grad_sign": ("dk = 1.0 - np.exp(d)", "dk = np.exp(d) - 1.0"),
    "kl_estimator_missing_one": ("k = np.exp(d) - d - 1.0", "k = np.exp(d) - d"),
    "ratio_inverted": ("r = np.exp(lp - old)", "r = np.exp(old - lp)"),
    "token_mean_over_batch": ("J = np.where(used, obj.sum(axis=1) / np.maximum(n, 1), 0.0)",
                              "J = np.where(used, obj.sum(axis=1) / max(int(n.sum()), 1), 0.0)"),
    "dpo_sigmoid_sign": ("g = beta * _sigmoid(-delta) / P", "g = beta * _sigmoid(delta) / P"),
    "dpo_pairs_reversed": ("delta = beta * ((pi[:P] - ref[:P]) - (pi[P:] - ref[P:]))",
                           "delta = beta * ((pi[P:] - ref[P:]) - (pi[:P] - ref[:P]))"),
    "kto_weights_swapped": ("lam = np.where(des, desirable_weight, undesirable_weight)",
                            "lam = np.where(des, undesirable_weight, desirable_weight)"),
    "kto_no_clamp": ("z0 = max(float(kl_ref), 0.0)", "z0 = float(kl_ref)"),
    "kto_grad_sign": ("dr = -lam * sx * (1.0 - sx) * np.where(des, beta, -beta) / n_seq",
                      "dr = lam * sx * (1.0 - sx) * np.where(des, beta, -beta) / n_seq"),
    "head_backward_as_nll": ('return fo.backward(hidden, weight, labels, ignore_index, "logprob", grad_out=g,',
                             'return fo.backward(hidden, weight, labels, ignore_index, "nll", grad_out=g,'),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not found once: {old!r}"
    modname = f"policy_oracle_mutant_{name}"
    mod = types.ModuleType(modname)
    sys.modules[modname] = mod          # dataclasses look the module up by name
    try:
        exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    finally:
        del sys.modules[modname]
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_policy_mutant_is_caught(name):
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
