"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them."""

import json
import os

import numpy as np
import pytest

from oracle import gated_rmsnorm
from tests import oracle_pins

HERE = os.path.dirname(os.path.abspath(__file__))
FIXTURE = json.load(open(os.path.join(HERE, "golden", "hand_example.json")))


def _make(mistake):
    def impl(q, k, v, alpha, beta, initial_state=None, scale=1.0):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        alpha, beta = np.asarray(alpha, np.float64), np.asarray(beta, np.float64)
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        S = np.zeros((B, H, dk, dv)) if initial_state is None else np.array(initial_state, np.float64)
        y = np.empty((B, T, H, dv))
        for t in range(T):
            ta = t - 1 if (mistake == "alpha_index_shift" and t > 0) else t
            a = alpha[:, ta, :, None, None]
            b = beta[:, t, :, None, None]
            kt, qt = k[:, t], q[:, t]
            S_old = S
            S_dec = a * S
            read_from = S if mistake == "read_before_decay" else S_dec
            if mistake == "transposed_read":
                recalled = np.matmul(read_from, kt[:, :, :, None])[..., 0]
            else:
                recalled = np.matmul(kt[:, :, None, :], read_from)[:, :, 0, :]
            e = v[:, t] - recalled
            write = kt[:, :, :, None] * e[:, :, None, :]
            if mistake == "write_sign":
                S = S_dec - b * write
            elif mistake == "dropped_beta":
                S = S_dec + write
            elif mistake == "decay_after_write":
                S = a * (S + b * (kt[:, :, :, None] * (v[:, t] - np.matmul(kt[:, :, None, :], S)[:, :, 0, :])[:, :, None, :]))
            elif mistake == "page3_compact_form":
                S = S_dec - b * kt[:, :, :, None] * np.matmul(kt[:, :, None, :], S)[:, :, 0, :][:, :, None, :] \
                    + b * kt[:, :, :, None] * v[:, t][:, :, None, :]
            else:
                S = S_dec + b * write
            read_out = S_old if mistake == "output_from_old_state" else S
            y[:, t] = scale * np.matmul(qt[:, :, None, :], read_out)[:, :, 0, :]
        return y, S
    return impl


MISTAKES = ["alpha_index_shift", "read_before_decay", "transposed_read", "write_sign",
            "dropped_beta", "decay_after_write", "page3_compact_form", "output_from_old_state"]


def _caught(impl):
    for pin in oracle_pins.RECURRENCE_PINS:
        try:
            if not pin(impl) < 1e-9:
                return True
        except (ValueError, IndexError):
            return True              # a shape mistake that cannot even run
    try:
        return not oracle_pins.pin_hand_example(impl, FIXTURE) < 1e-9
    except (ValueError, IndexError):
        return True


def test_unmutated_copy_passes():
    assert not _caught(_make(None))


@pytest.mark.parametrize("mistake", MISTAKES)
def test_pins_catch_planted_mistake(mistake):
    assert _caught(_make(mistake))


def _norm_mutant(kind):
    def f(y, z, w, eps):
        y, z, w = (np.asarray(x, np.float64) for x in (y, z, w))
        if kind == "layernorm":
            y = y - y.mean(axis=-1, keepdims=True)
        ms = np.mean(y * y, axis=-1, keepdims=True)
        gate = z / (1 + np.exp(-z)) if kind == "silu_gate" else 1 / (1 + np.exp(-z))
        scale = w if kind == "weight_not_zero_centred" else 1 + w
        denom = np.sqrt(ms) + eps if kind == "eps_outside_sqrt" else np.sqrt(ms + eps)
        return gate * y / denom * scale
    return f


@pytest.mark.parametrize("kind", ["layernorm", "silu_gate", "weight_not_zero_centred"])
def test_hand_values_catch_norm_mistakes(kind):
    f = _norm_mutant(kind)
    worst = 0.0
    for c in FIXTURE["gated_rmsnorm"]:
        out = f(c["y"], c["z"], c["weight"], c["eps"])
        worst = max(worst, float(np.max(np.abs(out - np.array(c["out"])))))
    assert worst > 1e-6


def test_torch_pin_catches_eps_placement():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((4, 16)) * 1e-2
    z = rng.standard_normal((4, 16))
    w = np.zeros(16)
    good = gated_rmsnorm(y, z, w, 1e-3)
    bad = _norm_mutant("eps_outside_sqrt")(y, z, w, 1e-3)
    assert np.max(np.abs(good - bad)) > 1e-3
