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


def chunked_backward(q, k, v, alpha, beta, dy, initial_state=None, d_final_state=None, scale=1.0, C=64,
                     log_floor=-30.0):
    """Float64 model of the chunked backward the GPU evaluates, in its four
    passes: per-chunk gates and C x C matrices (T, P, M); the forward walk of
    chunk-start states S_c (with E_c); the reverse walk of dS' (the gradient
    of each chunk's end state, with dR_c = T^T dE_c and dV); then per chunk the
    remaining gradients from S_c, dS'_c, E_c, dR_c.

    Chain rule through the chunk form above (n = C, tails padded with
    identity tokens):
        dE  = scale P^T dY + diag(lam) K dS',      dR = T^T dE,   dV = diag(beta) dR
        dS  = gamma_n dS' + scale Q^T diag(gamma) dY - K^T diag(beta gamma) dR
        X1 = dY S^T,  X2 = dR S^T,  X3 = E dS'^T,  X4 = dY E^T,  X5 = dR E^T
        dq  = scale gamma X1 + (dP o Gamma) K,            dP = scale X4 (i <= t)
        dk  = lam X3 - beta gamma X2 + (Dm + Dm^T) K + (dP o Gamma)^T Q,
              Dm = beta_t dA_ti Gamma_ti,  dA = -X5 (i < t)
        dbeta_t = dR_t.v_t - gamma_t k_t.X2_t + sum_i dA_ti M_ti,   M_ti = Gamma_ti k_t.k_i
        dgamma_t = scale q_t.X1_t - beta_t k_t.X2_t,   dlam_t = k_t.X3_t
        dg_t = gamma_t dgamma_t + rows(dP o P) - cols(dP o P) + rows(dA o A) - cols(dA o A)
               - lam_t dlam_t  (+ at t = n: sum lam dlam + gamma_n <dS', S>)
        dlog(alpha)_s = sum_{t >= s} dg_t;   dalpha = dlog(alpha) / alpha (0 where floored)
    """
    q, k, v, dy = (np.asarray(x, np.float64) for x in (q, k, v, dy))
    alpha, beta = np.asarray(alpha, np.float64), np.asarray(beta, np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    nch = (T + C - 1) // C
    Tp = nch * C

    def pad(x, fill=0.0):
        out = np.full((x.shape[0], Tp) + x.shape[2:], fill)
        out[:, :T] = x
        return out
    q_, k_, v_, dy_ = pad(q), pad(k), pad(v), pad(dy)
    a_, b_ = pad(alpha, 1.0), pad(beta)
    dq, dk_, dv_ = np.zeros_like(q_), np.zeros_like(k_), np.zeros_like(v_)
    da, db = np.zeros_like(a_), np.zeros_like(b_)
    dS0 = np.zeros((B, H, dk, dv))
    tril = np.tril(np.ones((C, C), bool))
    for b in range(B):
        for h in range(H):
            # pass 1: gates and chunk matrices
            chunks = []
            for c in range(nch):
                sl = slice(c * C, (c + 1) * C)
                Q, K = q_[b, sl, h], k_[b, sl, h]
                with np.errstate(divide="ignore"):
                    ell_raw = np.log(a_[b, sl, h])
                ell = np.maximum(ell_raw, log_floor)
                g = np.cumsum(ell)
                Gam = np.exp(np.where(tril, g[:, None] - g[None, :], -np.inf))
                M = np.tril(Gam * (K @ K.T), -1)
                A = b_[b, sl, h][:, None] * M
                Tm = np.linalg.inv(np.eye(C) + A)
                P = Gam * (Q @ K.T)
                chunks.append(dict(g=g, Gam=Gam, M=M, A=A, T=Tm, P=P, floored=ell_raw < log_floor))
            # pass 2: chunk-start states and E
            S = np.zeros((dk, dv)) if initial_state is None else np.array(initial_state[b, h], np.float64)
            for c, ch in enumerate(chunks):
                sl = slice(c * C, (c + 1) * C)
                K, V, be = k_[b, sl, h], v_[b, sl, h], b_[b, sl, h]
                gam, lam = np.exp(ch["g"]), np.exp(ch["g"][-1] - ch["g"])
                ch["S"] = S
                ch["E"] = ch["T"] @ (be[:, None] * (V - gam[:, None] * (K @ S)))
                S = gam[-1] * S + (lam[:, None] * K).T @ ch["E"]
            # pass 3: reverse walk of the state gradient
            dS = np.zeros((dk, dv)) if d_final_state is None else np.array(d_final_state[b, h], np.float64)
            for c in range(nch - 1, -1, -1):
                ch = chunks[c]
                sl = slice(c * C, (c + 1) * C)
                Q, K, dY, be = q_[b, sl, h], k_[b, sl, h], dy_[b, sl, h], b_[b, sl, h]
                gam, lam = np.exp(ch["g"]), np.exp(ch["g"][-1] - ch["g"])
                ch["dSend"] = dS
                dE = scale * ch["P"].T @ dY + lam[:, None] * (K @ dS)
                dR = ch["T"].T @ dE
                ch["dR"] = dR
                dv_[b, sl, h] = be[:, None] * dR
                dS = gam[-1] * dS + scale * Q.T @ (gam[:, None] * dY) - K.T @ ((be * gam)[:, None] * dR)
            dS0[b, h] = dS
            # pass 4: per-chunk gradients
            for c, ch in enumerate(chunks):
                sl = slice(c * C, (c + 1) * C)
                Q, K, V, dY, be = q_[b, sl, h], k_[b, sl, h], v_[b, sl, h], dy_[b, sl, h], b_[b, sl, h]
                g, Gam, M, A, P = ch["g"], ch["Gam"], ch["M"], ch["A"], ch["P"]
                S, dSe, E, dR = ch["S"], ch["dSend"], ch["E"], ch["dR"]
                gam, lam = np.exp(g), np.exp(g[-1] - g)
                X1, X2, X3 = dY @ S.T, dR @ S.T, E @ dSe.T
                X4, X5 = dY @ E.T, dR @ E.T
                dP = np.where(tril, scale * X4, 0.0)
                dA = np.tril(-X5, -1)
                DpG = dP * Gam
                Dm = be[:, None] * dA * Gam
                dq[b, sl, h] = scale * gam[:, None] * X1 + DpG @ K
                dk_[b, sl, h] = lam[:, None] * X3 - (be * gam)[:, None] * X2 + (Dm + Dm.T) @ K + DpG.T @ Q
                db[b, sl, h] = np.sum(dR * V, 1) - gam * np.sum(K * X2, 1) + np.sum(dA * M, 1)
                dgam = scale * np.sum(Q * X1, 1) - be * np.sum(K * X2, 1)
                dlam = np.sum(K * X3, 1)
                PP, AA = dP * P, dA * A
                dg = gam * dgam + PP.sum(1) - PP.sum(0) + AA.sum(1) - AA.sum(0) - lam * dlam
                dg[-1] += np.sum(lam * dlam) + gam[-1] * np.sum(dSe * S)
                dell = np.cumsum(dg[::-1])[::-1]
                da[b, sl, h] = np.where(ch["floored"], 0.0, dell / a_[b, sl, h])
    return (dq[:, :T], dk_[:, :T], dv_[:, :T], da[:, :T], db[:, :T], dS0)
