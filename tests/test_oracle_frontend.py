"""Pins of the float64 front-end oracle (oracle/frontend_ref.py) against values
worked by hand and against properties the definition fixes (causality, impulse
response, segment composition, scale invariance of the norm).  CPU only."""

import json
import os

import numpy as np
import pytest

from oracle import gdn_frontend, l2norm, short_conv, silu

HERE = os.path.dirname(os.path.abspath(__file__))
FIXTURE = json.load(open(os.path.join(HERE, "golden", "frontend_example.json")))


def _col(x):
    return np.asarray(x, dtype=np.float64).reshape(1, -1, 1, 1)


def test_conv_hand_example():
    c = FIXTURE["conv"]
    w = np.asarray(c["w"]).reshape(1, 1, -1)
    got = short_conv(_col(c["x"]), w)
    np.testing.assert_allclose(got.ravel(), c["conv_zero_history"], rtol=0, atol=1e-15)
    hist = np.asarray(c["history"]).reshape(1, -1, 1, 1)
    got = short_conv(_col(c["x"]), w, hist)
    np.testing.assert_allclose(got.ravel(), c["conv_with_history"], rtol=0, atol=1e-15)


def test_conv_impulse_response_is_the_filter():
    rng = np.random.default_rng(1)
    W, T = 4, 12
    w = rng.standard_normal((3, 5, W))
    x = np.zeros((1, T, 3, 5))
    x[0, 2] = 1.0
    out = short_conv(x, w)
    for m in range(T):
        expect = w[..., W - 1 - (m - 2)] if 0 <= m - 2 < W else np.zeros((3, 5))
        np.testing.assert_allclose(out[0, m], expect, rtol=0, atol=1e-15)


def test_conv_is_causal():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 20, 3, 8))
    w = rng.standard_normal((3, 8, 4))
    y0 = short_conv(x, w)
    x2 = x.copy()
    x2[:, 11:] = rng.standard_normal(x2[:, 11:].shape)
    y1 = short_conv(x2, w)
    np.testing.assert_array_equal(y0[:, :11], y1[:, :11])
    assert np.max(np.abs(y0[:, 11:] - y1[:, 11:])) > 1e-3


def test_conv_segments_compose():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 30, 3, 8))
    w = rng.standard_normal((3, 8, 4))
    whole = short_conv(x, w)
    a = short_conv(x[:, :13], w)
    b = short_conv(x[:, 13:], w, history=x[:, 10:13])
    np.testing.assert_allclose(np.concatenate([a, b], axis=1), whole, rtol=0, atol=1e-13)


def test_silu_and_norm_hand_values():
    c = FIXTURE["l2norm"]
    np.testing.assert_allclose(silu(np.asarray(c["x"])), c["silu"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(l2norm(silu(np.asarray(c["x"])), eps=0.0), c["l2norm_of_silu"], rtol=1e-15, atol=0)


def test_silu_identities():
    x = np.linspace(-8, 8, 101)
    assert silu(np.zeros(1))[0] == 0.0
    np.testing.assert_allclose(silu(-x), silu(x) - x, rtol=0, atol=1e-13)
    np.testing.assert_allclose(silu(np.asarray([40.0])), [40.0], rtol=1e-15)


def test_l2norm_unit_and_scale_invariant():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 7, 3, 16))
    n = l2norm(x, eps=0.0)
    np.testing.assert_allclose(np.linalg.norm(n, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(l2norm(3.5 * x, eps=0.0), n, rtol=1e-14)


def test_gate_hand_values():
    g = FIXTURE["gates"]
    T, H = 2, 2
    a = np.asarray(g["a_logit"]).reshape(1, T, 1).repeat(H, axis=2)
    b = np.asarray(g["b_logit"]).reshape(1, T, 1).repeat(H, axis=2)
    z = np.zeros((1, T, H, 4))
    w = np.zeros((H, 4, 1))
    # head h uses A[h], b_alpha[h]; token t uses a_logit[t]: the worked pairs are (t, h) = (0, 0) and (1, 1)
    _, _, _, alpha, beta = gdn_frontend(z, z, z, w, w, w, a, b, np.asarray(g["A"]), np.asarray(g["b_alpha"]))
    np.testing.assert_allclose(beta[0, :, 0], g["beta"], rtol=1e-15)
    np.testing.assert_allclose([alpha[0, 0, 0], alpha[0, 1, 1]], g["alpha"], rtol=1e-14)


def test_alpha_limits_and_monotone():
    a = np.linspace(-60, 30, 200).reshape(1, -1, 1)
    z = np.zeros((1, 200, 1, 2))
    w = np.zeros((1, 2, 1))
    _, _, _, alpha, _ = gdn_frontend(z, z, z, w, w, w, a, np.zeros_like(a), np.asarray([-1.0]), np.asarray([0.5]))
    alpha = alpha[0, :, 0]
    assert np.all(np.diff(alpha) <= 0) and np.all(np.diff(alpha[100:]) < 0)
    assert abs(alpha[0] - 1.0) < 1e-20 + np.exp(-1.0) * np.exp(-59.5) * 1.01
    assert np.all((alpha > 0) & (alpha <= 1))


def test_frontend_outputs_are_the_composition():
    rng = np.random.default_rng(5)
    B, T, H, dk, dv, W = 2, 9, 3, 8, 6, 4
    qp, kp = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk))
    vp = rng.standard_normal((B, T, H, dv))
    wq, wk, wv = rng.standard_normal((H, dk, W)), rng.standard_normal((H, dk, W)), rng.standard_normal((H, dv, W))
    a, b = rng.standard_normal((B, T, H)), rng.standard_normal((B, T, H))
    q, k, v, alpha, beta = gdn_frontend(qp, kp, vp, wq, wk, wv, a, b, rng.standard_normal(H), rng.standard_normal(H),
                                        eps=0.0)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-14)
    # v carries no norm; q is SiLU(conv) divided by its norm
    cq = silu(short_conv(qp, wq))
    np.testing.assert_allclose(q * np.linalg.norm(cq, axis=-1, keepdims=True), cq, rtol=0, atol=1e-13)
    np.testing.assert_allclose(v, silu(short_conv(vp, wv)), rtol=0, atol=0)


# ---- planted mistakes: each must be caught by one of the pins above ----

def _mutant_conv(kind):
    def conv(x, w, history=None):
        x, w = np.asarray(x, np.float64), np.asarray(w, np.float64)
        B, T, H, d = x.shape
        W = w.shape[-1]
        hist = np.zeros((B, W - 1, H, d)) if history is None else np.asarray(history, np.float64)
        padded = np.concatenate([hist, x], axis=1)
        out = np.zeros((B, T, H, d))
        for j in range(W):
            jj = W - 1 - j if kind == "reversed_taps" else j
            out += w[None, None, :, :, jj] * padded[:, j:j + T]
        if kind == "history_ignored":
            out = short_conv(x, w)
        return out
    return conv


@pytest.mark.parametrize("kind", ["reversed_taps", "history_ignored"])
def test_conv_pins_catch_planted_mistakes(kind):
    conv = _mutant_conv(kind)
    c = FIXTURE["conv"]
    w = np.asarray(c["w"]).reshape(1, 1, -1)
    bad = False
    bad |= not np.allclose(conv(_col(c["x"]), w).ravel(), c["conv_zero_history"])
    hist = np.asarray(c["history"]).reshape(1, -1, 1, 1)
    bad |= not np.allclose(conv(_col(c["x"]), w, hist).ravel(), c["conv_with_history"])
    assert bad


def test_gate_pins_catch_relu_for_softplus():
    g = FIXTURE["gates"]
    a = np.asarray(g["a_logit"]) + np.asarray(g["b_alpha"])
    alpha_relu = np.exp(-np.exp(np.asarray(g["A"])) * np.maximum(a, 0.0))
    assert not np.allclose(alpha_relu, g["alpha"])
