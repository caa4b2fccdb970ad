"""Plain float64 backward (reverse-mode gradients) of the gated delta rule.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
calls into this file, and this file never calls the HIP library.

Source: the forward is the delta form of "On the Design of Qwen3.8-Next
Architecture", slinene ai-papers-daily page, Module A (the same recurrence as
oracle/gdn_ref.py); the pages discuss the backward only as a training kernel
(the slinene page's FlashQLA paragraph), so the gradients below are the chain
rule applied to that forward, written out by hand step by step in reverse.

Per (b, h), the forward step t is
    S_dec = alpha_t S_{t-1};   e_t = v_t - S_dec^T k_t;
    S_t   = S_dec + beta_t k_t e_t^T;   y_t = scale S_t^T q_t,
and the loss is L = sum_t <dy_t, y_t> + <dS_T, S_T>.  With G the running
gradient of L with respect to the current state, going from t = T-1 down to 0:
    G      += scale q_t dy_t^T                 (y_t reads S_t)
    dq_t    = scale S_t dy_t
    de      = beta_t G^T k_t                   (S_t = S_dec + beta_t k_t e_t^T)
    dbeta_t = k_t^T G e_t
    dk_t    = beta_t G e_t - S_dec de          (write term, then the read in e_t)
    dv_t    = de
    G_dec   = G - k_t de^T                     (e_t = v_t - S_dec^T k_t)
    dalpha_t = <G_dec, S_{t-1}>
    G       = alpha_t G_dec                     (gradient of S_{t-1})
and dS_0 = G at the end.  States are recomputed forward from checkpoints taken
every ``checkpoint`` tokens (no reordering of the arithmetic: each recomputed
state is the same float64 sequence of operations as the first time).

Parity pins for this function live in tests/test_oracle_bwd.py.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _step(S, k_t, v_t, a_t, b_t):
    """One forward step on a batch of states [B, H, dk, dv] -> (S_dec, e, S_new)."""
    S_dec = a_t[:, :, None, None] * S
    e = v_t - np.matmul(k_t[:, :, None, :], S_dec)[:, :, 0, :]
    S_new = S_dec + b_t[:, :, None, None] * (k_t[:, :, :, None] * e[:, :, None, :])
    return S_dec, e, S_new


def gated_delta_backward(q, k, v, alpha, beta, dy, initial_state=None, d_final_state=None, scale=1.0,
                         checkpoint=64):
    """Gradients of L = sum <dy, y> + <dS_T, S_T> for the gated delta rule.

    Shapes: q, k [B, T, H, d_k]; v, dy [B, T, H, d_v]; alpha, beta [B, T, H];
    initial_state, d_final_state [B, H, d_k, d_v] or None (zeros).
    Returns (dq, dk, dv, dalpha, dbeta, d_initial_state), float64, with the
    shapes of q, k, v, alpha, beta and the state.
    """
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    alpha, beta = _f64(alpha), _f64(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if initial_state is None else _f64(initial_state).copy()

    # forward pass keeping only the state at every checkpoint
    starts = list(range(0, T, checkpoint))
    saved = []
    for c0 in starts:
        saved.append(S.copy())
        for t in range(c0, min(c0 + checkpoint, T)):
            _, _, S = _step(S, k[:, t], v[:, t], alpha[:, t], beta[:, t])

    G = np.zeros((B, H, dk, dv)) if d_final_state is None else _f64(d_final_state).copy()
    dq, dk_, dv_ = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dalpha, dbeta = np.zeros_like(alpha), np.zeros_like(beta)
    for c0, S_c in reversed(list(zip(starts, saved))):
        c1 = min(c0 + checkpoint, T)
        # recompute the states of this segment: prev[t - c0] = S_{t-1}
        prev, S = [], S_c
        for t in range(c0, c1):
            prev.append(S)
            _, _, S = _step(S, k[:, t], v[:, t], alpha[:, t], beta[:, t])
        for t in range(c1 - 1, c0 - 1, -1):
            S_prev = prev[t - c0]
            k_t, q_t, a_t, b_t = k[:, t], q[:, t], alpha[:, t], beta[:, t]
            S_dec, e, S_t = _step(S_prev, k_t, v[:, t], a_t, b_t)
            G = G + scale * (q_t[:, :, :, None] * dy[:, t][:, :, None, :])
            dq[:, t] = scale * np.matmul(S_t, dy[:, t][:, :, :, None])[..., 0]
            de = b_t[:, :, None] * np.matmul(k_t[:, :, None, :], G)[:, :, 0, :]          # beta G^T k
            Ge = np.matmul(G, e[:, :, :, None])[..., 0]                                    # G e  [B,H,dk]
            dbeta[:, t] = np.sum(k_t * Ge, axis=-1)
            dk_[:, t] = b_t[:, :, None] * Ge - np.matmul(S_dec, de[:, :, :, None])[..., 0]
            dv_[:, t] = de
            G_dec = G - k_t[:, :, :, None] * de[:, :, None, :]
            dalpha[:, t] = np.sum(G_dec * S_prev, axis=(-2, -1))
            G = a_t[:, :, None, None] * G_dec
    return dq, dk_, dv_, dalpha, dbeta, G
