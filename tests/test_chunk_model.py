"""The chunkwise form the prefill kernel uses reaches the oracle's result
(float64, up to rounding), for chunk sizes that do and do not divide T."""

import numpy as np
import pytest

from oracle import gated_delta_recurrence
from tests.chunk_model import chunked_recurrence
from tests.oracle_pins import _rand_inputs
from workloads import config_prefill_inputs


@pytest.mark.parametrize("C", [1, 7, 16, 64])
def test_chunked_equals_oracle(C):
    rng = np.random.default_rng(100 + C)
    q, k, v, a, b, S0 = _rand_inputs(rng, B=2, T=150, H=2, dk=6, dv=5)
    y, S = gated_delta_recurrence(q, k, v, a, b, S0, scale=0.5)
    yc, Sc = chunked_recurrence(q, k, v, a, b, S0, scale=0.5, C=C)
    assert np.max(np.abs(yc - y)) < 1e-11
    assert np.max(np.abs(Sc - S)) < 1e-11


def test_chunked_equals_oracle_on_config0():
    d = config_prefill_inputs(0)
    y, S = gated_delta_recurrence(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    yc, Sc = chunked_recurrence(d["q"], d["k"], d["v"], d["alpha"], d["beta"], C=64)
    assert np.max(np.abs(yc - y)) < 1e-12
    assert np.max(np.abs(Sc - S)) < 1e-12


def test_chunked_log_floor_alpha_zero():
    """A floored log-decay reproduces alpha = 0 to far below any tolerance."""
    rng = np.random.default_rng(7)
    q, k, v, a, b, S0 = _rand_inputs(rng, B=1, T=40, H=1, dk=4, dv=3)
    a[0, [3, 17, 18, 39], 0] = 0.0
    y, S = gated_delta_recurrence(q, k, v, a, b, S0)
    yc, Sc = chunked_recurrence(q, k, v, a, b, S0, C=16, log_floor=-80.0)
    assert np.max(np.abs(yc - y)) < 1e-10
    assert np.max(np.abs(Sc - S)) < 1e-10


@pytest.mark.parametrize("C,T", [(64, 150), (16, 40), (8, 8), (7, 23)])
def test_chunked_backward_equals_oracle_backward(C, T):
    """The four-pass chunked backward (what the GPU evaluates) reaches the
    token-by-token backward oracle's gradients, ragged tails included."""
    from oracle import gated_delta_backward
    from tests.chunk_model import chunked_backward
    rng = np.random.default_rng(200 + C)
    q, k, v, a, b, S0 = _rand_inputs(rng, B=2, T=T, H=2, dk=6, dv=5)
    dy = rng.standard_normal(v.shape)
    dST = rng.standard_normal(S0.shape)
    ref = gated_delta_backward(q, k, v, a, b, dy, S0, dST, scale=0.8)
    got = chunked_backward(q, k, v, a, b, dy, S0, dST, scale=0.8, C=C)
    for name, x, r in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dS0"), got, ref):
        np.testing.assert_allclose(x, r, rtol=0, atol=1e-10 * (1 + np.max(np.abs(r))), err_msg=name)
