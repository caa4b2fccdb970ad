"""The operand-precision plan of the bf16 prefill, checked in float64
(tests/precision_model.py against the oracle): with every intermediate the
kernels round rounded to fp16 and a float32 state and y, the error stays well
inside the 2e-2 bound; rounding the same intermediates to bf16 instead, or
storing y as bf16, exceeds it.  Inputs: 1024 tokens, 3 heads, d = 128, drawn
as the 4K and 32K workloads (A = -1 and -2)."""

import pytest

from oracle import gated_delta_recurrence, rel_err
from tests.precision_model import OPERANDS, chunked_with_rounding
from workloads import config_prefill_inputs

BOUND = 2e-2
INTERMEDIATES = [o for o in OPERANDS if o != "y"]


def _errors(cfg, plan):
    d = config_prefill_inputs(cfg, T=1024, H=3, B=1)
    y_ref, S_ref = gated_delta_recurrence(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    y, S = chunked_with_rounding(d["q"], d["k"], d["v"], d["alpha"], d["beta"], plan)
    return rel_err(y, y_ref), rel_err(S, S_ref)


@pytest.mark.parametrize("cfg", [1, 2])
def test_model_without_rounding_is_the_oracle(cfg):
    ey, eS = _errors(cfg, {})
    assert ey < 1e-10 and eS < 1e-10


@pytest.mark.parametrize("cfg", [1, 2])
def test_fp16_operands_fit_the_bf16_bound_with_margin(cfg):
    ey, eS = _errors(cfg, {o: "fp16" for o in INTERMEDIATES})
    assert ey < BOUND / 2 and eS < BOUND / 2, (ey, eS)


@pytest.mark.parametrize("cfg", [1, 2])
def test_bf16_operands_exceed_the_bound(cfg):
    ey, _ = _errors(cfg, {o: "bf16" for o in INTERMEDIATES})
    assert ey > BOUND, ey


def test_bf16_y_alone_exceeds_the_bound():
    ey, eS = _errors(1, {"y": "bf16"})
    assert ey > BOUND and eS < 1e-10, (ey, eS)
