"""Plant plausible mistakes in copies of the oracle; some pin must catch each one."""
import os
import sys
import types
import warnings

import pytest

import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "flce_oracle.py")

MUTANTS = {
    "no_max_shift": ("return m + np.log(np.exp(z - m[:, None]).sum(axis=1))",
                     "return np.log(np.exp(z).sum(axis=1))"),
    "nll_sign": ("nll = lse - zy", "nll = zy - lse"),
    "label_off_by_one": ("zy[r0 + rows] = z[rows, labels[r0 + rows]]",
                         "zy[r0 + rows] = z[rows, (labels[r0 + rows] + 1) % V]"),
    "mean_over_all_tokens": ("mean = float(out[valid].sum() / n_valid) if n_valid else 0.0",
                             "mean = float(out.sum() / T)"),
    "dropped_onehot": ("g[rows, labels[rows]] -= 1.0", "pass"),
    "logprob_grad_sign": ("    if mode == \"logprob\":\n        g = -g\n", ""),
    "ignored_tokens_get_grad": ("return np.where(valid, g, 0.0)", "return g"),
    "mean_grad_over_T": ("g = np.full(valid.shape, gm / n_valid if n_valid else 0.0)",
                         "g = np.full(valid.shape, gm / len(valid))"),
    "bf16_decode_shift": ("f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)",
                          "f32 = (b.astype(np.uint32) << np.uint32(15)).view(np.float32)"),
    "dh_uses_softmax_only": ("dh[r0:r1] = g @ w", "dh[r0:r1] = np.exp(z - l[:, None]) @ w"),
    "dw_transposed_rows": ("dw += g.T @ h[r0:r1]", "dw += (g.T @ h[r0:r1])[::-1]"),
    # logit transforms
    "softcap_no_chain_rule": ("d = d * (1.0 - t * t)", "d = d * 1.0"),
    "softcap_without_division": ("t = np.tanh(x / self.softcap)", "t = np.tanh(x)"),
    "temperature_multiplies": ("            x = x / self.temperature\n",
                               "            x = x * self.temperature\n"),
    "temperature_before_cap": ("            t = np.tanh(x / self.softcap)\n            x = self.softcap * t\n",
                               "            t = np.tanh(x / self.temperature / self.softcap)\n"
                               "            x = self.softcap * t * self.temperature\n"),
    "divide_multiplies": ("            x = x / self.scale_divide\n", "            x = x * self.scale_divide\n"),
    "weight_rows_drop_chain": ("    if dz is not None:\n        g *= dz\n", ""),
    # row-blocked loops and the page's chunk multiplier
    "block_label_offset_dropped": ("zy[r0 + rows] = z[rows, labels[r0 + rows]]",
                                   "zy[rows] = z[rows, labels[r0 + rows]]"),
    "block_given_lse_offset_dropped": (
        "l = logsumexp_rows(z) if lse is None else np.asarray(lse[r0:r1], dtype=np.float64)",
        "l = logsumexp_rows(z) if lse is None else np.asarray(lse[:r1 - r0], dtype=np.float64)"),
    "block_scale_offset_dropped": ("g = grad_logits(z, l, labels[r0:r1], c[r0:r1], dz)",
                                   "g = grad_logits(z, l, labels[r0:r1], c[:r1 - r0], dz)"),
    "multiplier_divisor_2048": ("return max(4, context // 4096)", "return max(4, context // 2048)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not found once: {old!r}"
    modname = f"flce_oracle_mutant_{name}"
    mod = types.ModuleType(modname)
    sys.modules[modname] = mod          # dataclasses look the module up by name
    try:
        exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    finally:
        del sys.modules[modname]
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
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
