"""The oracle against facts fixed by the pages and by mathematics (CPU only)."""
import json
import math
import os

import pytest

import oracle_pins as pins
from oracle import flce_oracle as o

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(o)


def _pages():
    with open(os.path.join(HERE, "golden", "pages_memory.json")) as f:
        return json.load(f)


def test_logit_memory_formulas():
    """Equations 1-3 of the Unsloth page: the formulas, and where the printed values stand."""
    p = _pages()
    e1 = p["eq1_example"]
    b, c, v = e1["batch"], e1["context"], e1["vocab"]
    # the formula has no byte factor: 1 byte per element, in GiB
    assert o.logit_memory_eq1(b, c, v) == 3.90625
    assert o.logit_memory_eq1(b, c, v, 2) == 7.8125            # bf16
    assert o.logit_memory_eq1(b, c, v, 4) == 15.625            # fp32 chunk logits
    assert o.logit_memory_eq2(c, v) == o.logit_memory_eq1(b, c, v) / b
    mult = o.default_multiplier(c)
    assert mult == 4
    assert o.logit_memory_eq3(c, v, mult) == o.logit_memory_eq2(c, v) / 4
    # The printed chain 3.3 -> 0.83 -> 0.207 divides by 4 twice, as the formulas do,
    # but starts from 3.3 where Equation 1 gives 3.906: a page inconsistency, recorded.
    assert abs(p["eq2_example"]["printed_gb"] - e1["printed_gb"] / 4) < 0.01
    assert abs(p["eq3_example"]["printed_gb"] - p["eq2_example"]["printed_gb"] / 4) < 0.001
    assert abs(o.logit_memory_eq1(b, c, v) - e1["printed_gb"]) > 0.5


def test_hidden_state_and_fp32_copy_figures():
    p = _pages()
    hs = p["hidden_states_example"]
    full = o.hidden_memory(hs["batch"], hs["context"], hs["hidden"])
    assert round(full) == hs["printed_gb"]
    assert round(full / hs["batch"], 3) == hs["printed_chunked_gb"]
    cp = p["fp32_lm_head_copy"]
    nbytes = cp["vocab"] * cp["hidden"] * cp["bytes_per_elem"]
    assert nbytes == 2_034_237_440
    assert round(nbytes / 1e9, 2) == cp["printed_gb"]          # decimal GB on that page


def test_zero_weight_ln_v_values():
    """ln V for the workload vocabularies (the W = 0 closed form)."""
    assert math.isclose(math.log(1000), 6.907755, abs_tol=1e-6)
    assert math.isclose(math.log(248320), 12.422474, abs_tol=1e-6)
    assert math.isclose(math.log(151936), 11.931215, abs_tol=1e-6)
    assert math.isclose(math.log(128000), 11.759786, abs_tol=1e-6)
