"""Pins of the float64 backward oracle (oracle/bwd_ref.py): central finite
differences of the (separately pinned) forward oracle, torch autograd through
an independent torch float64 forward, closed forms at beta = 0, and planted
mistakes that the finite-difference pin must catch.  CPU only."""

import numpy as np
import pytest
import torch

from oracle import gated_delta_backward, gated_delta_recurrence


def _inputs(seed, B=1, T=5, H=2, dk=3, dv=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    a = rng.uniform(0.3, 0.99, (B, T, H))
    b = rng.uniform(0.05, 0.95, (B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    dy = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    return q, k, v, a, b, S0, dy, dST


def _loss(q, k, v, a, b, S0, dy, dST, scale):
    y, S = gated_delta_recurrence(q, k, v, a, b, S0, scale=scale)
    return float(np.sum(y * dy) + np.sum(S * dST))


def _finite_difference_check(backward, seed=1, scale=0.7, h=1e-6):
    q, k, v, a, b, S0, dy, dST = _inputs(seed)
    grads = backward(q, k, v, a, b, dy, S0, dST, scale=scale)
    args = [q, k, v, a, b, S0]
    worst = 0.0
    for which, g in zip(range(6), grads):
        x = args[which]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(*args, dy, dST, scale)
            x[idx] = old - h
            lm = _loss(*args, dy, dST, scale)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        worst = max(worst, float(np.max(np.abs(fd - g)) / (np.max(np.abs(fd)) + 1e-30)))
    return worst


def test_matches_central_finite_differences():
    assert _finite_difference_check(gated_delta_backward) < 1e-7


def _torch_forward(q, k, v, a, b, S0, scale):
    """The delta form written with torch ops (autograd differentiates it)."""
    B, T, H, dk = q.shape
    S = S0
    ys = []
    for t in range(T):
        S_dec = a[:, t, :, None, None] * S
        e = v[:, t] - torch.einsum("bhk,bhkv->bhv", k[:, t], S_dec)
        S = S_dec + b[:, t, :, None, None] * torch.einsum("bhk,bhv->bhkv", k[:, t], e)
        ys.append(scale * torch.einsum("bhk,bhkv->bhv", q[:, t], S))
    return torch.stack(ys, dim=1), S


@pytest.mark.parametrize("checkpoint", [64, 7, 1])
def test_matches_torch_autograd(checkpoint):
    q, k, v, a, b, S0, dy, dST = _inputs(2, B=2, T=70, H=2, dk=5, dv=4)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, a, b, S0)]
    y, S = _torch_forward(*ts, scale=1.3)
    (torch.sum(y * torch.from_numpy(dy)) + torch.sum(S * torch.from_numpy(dST))).backward()
    grads = gated_delta_backward(q, k, v, a, b, dy, S0, dST, scale=1.3, checkpoint=checkpoint)
    for name, t, g in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dS0"), ts, grads):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=0, atol=1e-10, err_msg=name)


def test_checkpoint_spacing_does_not_change_results():
    q, k, v, a, b, S0, dy, dST = _inputs(3, B=1, T=40, H=2, dk=4, dv=3)
    r1 = gated_delta_backward(q, k, v, a, b, dy, S0, dST, checkpoint=64)
    r2 = gated_delta_backward(q, k, v, a, b, dy, S0, dST, checkpoint=6)
    for x1, x2 in zip(r1, r2):
        np.testing.assert_array_equal(x1, x2)


def test_pure_decay_closed_form():
    """beta = 0: y_t = scale G_t S0^T q_t with G_t the running product of alphas,
    so dq_t = scale G_t S0 dy_t, dv = 0 and dS0 = sum_t scale G_t q_t dy_t^T + G_T dS_T."""
    q, k, v, a, _, S0, dy, dST = _inputs(4, B=2, T=9, H=3, dk=4, dv=3)
    b = np.zeros_like(a)
    dq, _, dv, _, _, dS0 = gated_delta_backward(q, k, v, a, b, dy, S0, dST, scale=0.5)
    G = np.cumprod(a, axis=1)
    np.testing.assert_allclose(dq, 0.5 * G[..., None] * np.einsum("bhkv,bthv->bthk", S0, dy), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(dv, np.zeros_like(dv))
    expect = 0.5 * np.einsum("bth,bthk,bthv->bhkv", G, q, dy) + G[:, -1, :, None, None] * dST
    np.testing.assert_allclose(dS0, expect, rtol=0, atol=1e-12)


def test_zero_cotangent_gives_zero_gradients():
    q, k, v, a, b, S0, dy, dST = _inputs(5)
    for g in gated_delta_backward(q, k, v, a, b, np.zeros_like(dy), S0, None):
        np.testing.assert_array_equal(g, np.zeros_like(g))


def _mutant(mistake):
    """A copy of the backward with one plausible mistake planted."""
    def backward(q, k, v, alpha, beta, dy, S0, dST, scale=1.0):
        B, T, H, dk = q.shape
        S = S0.copy()
        states = [S]
        for t in range(T):
            S_dec = alpha[:, t, :, None, None] * S
            e = v[:, t] - np.einsum("bhk,bhkv->bhv", k[:, t], S_dec)
            S = S_dec + beta[:, t, :, None, None] * np.einsum("bhk,bhv->bhkv", k[:, t], e)
            states.append(S)
        G = dST.copy()
        out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(alpha), np.zeros_like(beta)]
        for t in range(T - 1, -1, -1):
            S_prev, S_t = states[t], states[t + 1]
            a_t, b_t, k_t = alpha[:, t], beta[:, t], k[:, t]
            S_dec = a_t[:, :, None, None] * S_prev
            e = v[:, t] - np.einsum("bhk,bhkv->bhv", k_t, S_dec)
            if mistake != "output_grad_after_state_grad":
                G = G + scale * np.einsum("bhk,bhv->bhkv", q[:, t], dy[:, t])
            out[0][:, t] = scale * np.einsum("bhkv,bhv->bhk", S_t, dy[:, t])
            de = b_t[:, :, None] * np.einsum("bhk,bhkv->bhv", k_t, G)
            Ge = np.einsum("bhkv,bhv->bhk", G, e)
            out[4][:, t] = np.sum(k_t * Ge, axis=-1) * (-1 if mistake == "beta_sign" else 1)
            read = 0 if mistake == "dropped_read_term" else np.einsum("bhkv,bhv->bhk", S_dec, de)
            out[1][:, t] = b_t[:, :, None] * Ge - read
            out[2][:, t] = de
            G_dec = G - np.einsum("bhk,bhv->bhkv", k_t, de)
            out[3][:, t] = np.sum(G_dec * (S_t if mistake == "alpha_from_new_state" else S_prev), axis=(-2, -1))
            if mistake == "output_grad_after_state_grad":
                G_dec = G_dec + scale * np.einsum("bhk,bhv->bhkv", q[:, t], dy[:, t])
            G = G_dec if mistake == "undecayed_state_grad" else a_t[:, :, None, None] * G_dec
        return (*out, G)
    return backward


@pytest.mark.parametrize("mistake", ["dropped_read_term", "beta_sign", "alpha_from_new_state",
                                     "undecayed_state_grad", "output_grad_after_state_grad"])
def test_finite_differences_catch_planted_mistakes(mistake):
    assert _finite_difference_check(_mutant(mistake)) > 1e-3


def test_unmutated_copy_passes():
    assert _finite_difference_check(_mutant(None)) < 1e-7
