"""Float64 model of the bf16 prefill's operand precisions.

The bf16 prefill evaluates the chunk form (C = 64) with fp16 MFMA operands,
float32 accumulation, a float32 state and float32 y.  This model follows the
same data flow in float64 and rounds every value at the point where the
kernels round it, with the rounding chosen per operand; comparing the result
with the token-by-token oracle gives the error budget of each choice:

    q, k, v          inputs converted to the operand type
    T' = T diag(b)   the chunk inverse as stored by the chunk-parallel pass
    S                the state's operand copy (the float32 master stays exact)
    R = V - g K S    the residual, operand of T' R
    E = T' R         the misses, operand of P E (output) and, times d, of K^T D E
    P                the decay-masked Q K^T, operand of P E
    y                the output as stored

Test-side only (the HIP library shares nothing with it).
"""

import numpy as np

from workloads import round_to_bf16


def round_fp16(x):
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def round_bf16(x):
    return round_to_bf16(np.asarray(x, np.float64)).astype(np.float64)


def exact(x):
    return np.asarray(x, np.float64)


ROUNDING = {"fp16": round_fp16, "bf16": round_bf16, "exact": exact}
OPERANDS = ("qkv", "T", "S", "R", "E", "P", "y")


def chunked_with_rounding(q, k, v, alpha, beta, plan, C=64):
    """The chunk form of the recurrence with the roundings of `plan`, a dict
    mapping each name of OPERANDS to "fp16", "bf16" or "exact" (missing names
    are exact).  Shapes as the oracle's; zero initial state.  Returns (y, S)."""
    r = {name: ROUNDING[plan.get(name, "exact")] for name in OPERANDS}
    q, k, v = (r["qkv"](x) for x in (q, k, v))
    alpha, beta = np.asarray(alpha, np.float64), np.asarray(beta, np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    y = np.empty((B, T, H, dv))
    S_out = np.empty((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv))
            for c0 in range(0, T, C):
                n = min(C, T - c0)
                Q, K, V = q[b, c0:c0 + n, h], k[b, c0:c0 + n, h], v[b, c0:c0 + n, h]
                be = beta[b, c0:c0 + n, h]
                g = np.cumsum(np.log(alpha[b, c0:c0 + n, h]))
                lower = np.tril(np.ones((n, n), bool))
                Gam = np.exp(np.where(lower, g[:, None] - g[None, :], -np.inf))
                A = np.tril(be[:, None] * Gam * (K @ K.T), -1)
                Tp = r["T"](np.linalg.inv(np.eye(n) + A) * be[None, :])
                gam = np.exp(g)
                Sq = r["S"](S)
                R = r["R"](V - gam[:, None] * (K @ Sq))
                E = Tp @ R
                P = r["P"](Gam * (Q @ K.T))
                y[b, c0:c0 + n, h] = r["y"](gam[:, None] * (Q @ Sq) + P @ r["E"](E))
                d = np.exp(g[-1] - g)
                S = gam[-1] * S + K.T @ r["E"](d[:, None] * E)
            S_out[b, h] = S
    return y, S_out
