"""Float64 model of the chunkwise (WY / UT-transform) form of the gated delta
rule: the algebra the prefill kernel evaluates, written with numpy so that it
can be compared against the token-by-token oracle.  Test-side only; it shares
nothing with the HIP library.

Derivation (from the delta form on the slinene page, Module A).  Inside a
chunk of n tokens that starts from state S, write g_t = sum_{i<=t} log alpha_i,
gamma_t = exp(g_t) and Gamma_ti = exp(g_t - g_i) for i <= t.  With
e_t = beta_t (v_t - alpha_t S_{t-1}^T k_t) the state after token t is
S_t = gamma_t S + sum_{i<=t} Gamma_ti k_i e_i^T, so

    (I + A) E = diag(beta) V - diag(beta gamma) K S,
    A_ti = beta_t Gamma_ti k_t.k_i  (i < t), zero elsewhere,

and with T = (I + A)^-1:
    E  = T diag(beta) V - T diag(beta gamma) K S
    Y  = diag(gamma) Q S + P E,          P_ti = Gamma_ti q_t.k_i  (i <= t)
    S' = gamma_n S + K^T diag(exp(g_n - g)) E.
"""

import numpy as np


def chunked_recurrence(q, k, v, alpha, beta, initial_state=None, scale=1.0, C=64,
                       log_floor=None):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    alpha, beta = np.asarray(alpha, np.float64), np.asarray(beta, np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    y = np.empty((B, T, H, dv))
    S_out = np.empty((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else np.array(initial_state[b, h], np.float64)
            for c0 in range(0, T, C):
                n = min(C, T - c0)
                Q, K, V = q[b, c0:c0 + n, h], k[b, c0:c0 + n, h], v[b, c0:c0 + n, h]
                be = beta[b, c0:c0 + n, h]
                with np.errstate(divide="ignore"):
                    ell = np.log(alpha[b, c0:c0 + n, h])
                if log_floor is not None:
                    ell = np.maximum(ell, log_floor)
                g = np.cumsum(ell)
                lower = np.tril(np.ones((n, n), bool))
                diff = np.where(lower, g[:, None] - g[None, :], -np.inf)
                Gam = np.exp(diff)                      # zero above the diagonal
                A = np.tril(be[:, None] * Gam * (K @ K.T), -1)
                Tm = np.linalg.inv(np.eye(n) + A)
                gam = np.exp(g)
                E = Tm @ (be[:, None] * V) - Tm @ ((be * gam)[:, None] * K) @ S
                P = Gam * (Q @ K.T)
                y[b, c0:c0 + n, h] = scale * (gam[:, None] * (Q @ S) + P @ E)
                S = gam[-1] * S + (K * np.exp(g[-1] - g)[:, None]).T @ E
            S_out[b, h] = S
    return y, S_out
