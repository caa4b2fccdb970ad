"""The float64 oracle against what the pages and the mathematics fix."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import gated_delta_decode_step, gated_delta_recurrence, gated_rmsnorm, rel_err
from tests import oracle_pins

HERE = os.path.dirname(os.path.abspath(__file__))
FIXTURE = json.load(open(os.path.join(HERE, "golden", "hand_example.json")))
TOL = 1e-12


@pytest.mark.parametrize("pin", oracle_pins.RECURRENCE_PINS, ids=lambda f: f.__name__)
def test_recurrence_pin(pin):
    assert pin(gated_delta_recurrence) < TOL


def test_hand_example():
    assert oracle_pins.pin_hand_example(gated_delta_recurrence, FIXTURE) < TOL


def test_hand_example_page3_form_differs():
    """The slinene page's printed compact form leaves (-1.75, 4) after t = 3 in
    the hand example, where the delta form leaves (0, 4)."""
    r = FIXTURE["recurrence"]
    S = np.zeros((2, 1))
    for t in range(4):
        k = np.array(r["k"][t], dtype=np.float64)
        a, b = r["alpha"][t], r["beta"][t]
        S = (a * np.eye(2) - b * np.outer(k, k)) @ S + b * np.outer(k, r["v"][t])
    assert np.allclose(S, np.array(r["slinene_compact_form_state_after_t3"]))
    assert not np.allclose(S, np.array(r["final_state"]))


def test_scale_is_linear_on_outputs_only():
    rng = np.random.default_rng(5)
    q, k, v, a, b, S0 = oracle_pins._rand_inputs(rng)
    y1, S1 = gated_delta_recurrence(q, k, v, a, b, S0)
    y2, S2 = gated_delta_recurrence(q, k, v, a, b, S0, scale=0.25)
    assert np.max(np.abs(y2 - 0.25 * y1)) < TOL
    assert np.max(np.abs(S2 - S1)) == 0.0


def test_decode_steps_equal_recurrence():
    rng = np.random.default_rng(6)
    q, k, v, a, b, S0 = oracle_pins._rand_inputs(rng, T=7)
    y, S = gated_delta_recurrence(q, k, v, a, b, S0)
    St = S0
    for t in range(q.shape[1]):
        yt, St_new = gated_delta_decode_step(q[:, t], k[:, t], v[:, t], a[:, t], b[:, t], St)
        assert np.max(np.abs(yt - y[:, t])) < TOL
        St = St_new
    assert np.max(np.abs(St - S)) < TOL


def test_decode_does_not_modify_input_state():
    rng = np.random.default_rng(7)
    q, k, v, a, b, S0 = oracle_pins._rand_inputs(rng, T=1)
    keep = S0.copy()
    gated_delta_decode_step(q[:, 0], k[:, 0], v[:, 0], a[:, 0], b[:, 0], S0)
    assert np.array_equal(S0, keep)


def test_zero_length_sequence():
    q = np.zeros((1, 0, 2, 4))
    v = np.zeros((1, 0, 2, 3))
    a = np.zeros((1, 0, 2))
    S0 = np.arange(24.0).reshape(1, 2, 4, 3)
    y, S = gated_delta_recurrence(q, q, v, a, a, S0)
    assert y.shape == (1, 0, 2, 3)
    assert np.array_equal(S, S0)


def test_alpha_zero_forgets_everything_before():
    """alpha_t = 0 wipes the state: the result equals a fresh start at t."""
    rng = np.random.default_rng(8)
    q, k, v, a, b, S0 = oracle_pins._rand_inputs(rng, T=8)
    a[:, 3] = 0.0
    y, S = gated_delta_recurrence(q, k, v, a, b, S0)
    y2, S2 = gated_delta_recurrence(q[:, 3:], k[:, 3:], v[:, 3:], a[:, 3:], b[:, 3:], None)
    assert np.max(np.abs(y[:, 3:] - y2)) < TOL
    assert np.max(np.abs(S - S2)) < TOL


# ---- gated RMSNorm epilogue -------------------------------------------------

@pytest.mark.parametrize("case", range(len(FIXTURE["gated_rmsnorm"])))
def test_gated_rmsnorm_hand_values(case):
    c = FIXTURE["gated_rmsnorm"][case]
    out = gated_rmsnorm(np.array(c["y"]), np.array(c["z"]), np.array(c["weight"]), c["eps"])
    assert np.max(np.abs(out - np.array(c["out"]))) < 1e-15


def test_gated_rmsnorm_matches_torch_rms_norm():
    """With weight 1 + w this is torch's RMSNorm times torch's sigmoid (float64 CPU)."""
    rng = np.random.default_rng(9)
    y = rng.standard_normal((5, 3, 16)) * 2.0
    z = rng.standard_normal((5, 3, 16))
    w = rng.standard_normal(16) * 0.1
    eps = 1e-6
    ref = (torch.nn.functional.rms_norm(torch.tensor(y), [16], torch.tensor(1.0 + w), eps)
           * torch.sigmoid(torch.tensor(z))).numpy()
    assert np.max(np.abs(gated_rmsnorm(y, z, w, eps) - ref)) < 1e-13


def test_gated_rmsnorm_closed_forms():
    rng = np.random.default_rng(10)
    y = rng.standard_normal((7, 32))
    eps = 1e-3
    out = gated_rmsnorm(y, np.zeros_like(y), None, eps)
    m = np.mean(y * y, axis=-1)
    # z = 0 gives half the plain norm, whose RMS is sqrt(m / (m + eps))
    assert np.max(np.abs(np.sqrt(np.mean((2 * out) ** 2, axis=-1)) - np.sqrt(m / (m + eps)))) < 1e-14
    # the gate is a sigmoid: bounded in (0, 1), so |o| <= |y / rms|
    big = gated_rmsnorm(y, np.full_like(y, 40.0), None, 0.0)
    assert np.max(np.abs(big - y / np.sqrt(m)[:, None])) < 1e-12
    assert np.all(np.abs(gated_rmsnorm(y, rng.standard_normal(y.shape) * 5, None, 0.0))
                  <= np.abs(y / np.sqrt(m)[:, None]) + 1e-15)
    # no mean subtraction: a constant row normalises to all ones
    c = gated_rmsnorm(np.full((1, 8), -3.0), np.full((1, 8), 40.0), None, 0.0)
    assert np.max(np.abs(c + 1.0)) < 1e-12


def test_rel_err():
    ref = np.array([3.0, -4.0])
    assert rel_err(ref, ref) == 0.0
    assert abs(rel_err(ref + np.array([0.0, 0.1]), ref) - 0.1 / np.sqrt(12.5)) < 1e-15


def test_oracle_package_header_says_test_infrastructure():
    assert "TEST INFRASTRUCTURE ONLY" in oracle.__doc__
