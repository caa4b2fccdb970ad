"""Plain float64 definition of multi-token (speculative) decode for the GDN state.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
calls into this file, and this file never calls the HIP library.

Source: the rainbus digest of "On the Design of Qwen3.8-Next Architecture"
(its prerequisites section, the paragraph on multi-token prediction and
speculative decoding: a light module drafts several tokens at once, which the
main model then verifies in parallel) together with the delta form of
the recurrence on the slinene ai-papers-daily page, Module A.  A draft block
of K tokens is K ordinary recurrence steps taken from a live state; when only
the first j drafts are accepted, the live state must become the state after
those j steps and nothing else.

Two operations, each written out token by token:

  mtp_verify:  from the live state S_0, for t = 1 .. K
        S_dec = alpha_t S_{t-1}
        e_t   = v_t - S_dec^T k_t          (the miss, as in Module A)
        S_t   = S_dec + beta_t k_t e_t^T
        y_t   = scale * S_t^T q_t
     returns every y_t, every e_t and every prefix state S_t; the live state
     itself is left alone.

  mtp_commit:  given the e_t of a verified block and the number j of accepted
     drafts, replay the first j writes on the live state:
        S <- alpha_t S + beta_t k_t e_t^T,   t = 1 .. j.
     The result is exactly the prefix state S_j of the verify call (the e_t
     already hold the misses of that block), so no prefix state has to be kept
     in memory to roll back.

Readings: the pages name the drafting scheme but print
no kernel; the draft block uses the same q, k, v, alpha, beta per token as a
prefill, laid out [N, K, H, ...] (sequence, draft position, head), and j runs
from 0 (reject all) to K (accept all).  Parity pins live in
tests/test_oracle_mtp.py.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def mtp_verify(q, k, v, alpha, beta, state, scale=1.0):
    """Verify a block of K draft tokens from the live states.

    Shapes: q, k [N, K, H, d_k]; v [N, K, H, d_v]; alpha, beta [N, K, H];
    state [N, H, d_k, d_v].  Returns (y [N, K, H, d_v], e [N, K, H, d_v],
    prefix_states [N, K, H, d_k, d_v]) in float64; ``state`` is not modified.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta, S0 = _f64(alpha), _f64(beta), _f64(state)
    N, K, H, dk = q.shape
    dv = v.shape[-1]
    y = np.empty((N, K, H, dv))
    e = np.empty((N, K, H, dv))
    prefix = np.empty((N, K, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = S0[n, h].copy()
            for t in range(K):
                S_dec = alpha[n, t, h] * S
                miss = v[n, t, h] - S_dec.T @ k[n, t, h]
                S = S_dec + beta[n, t, h] * np.outer(k[n, t, h], miss)
                e[n, t, h] = miss
                y[n, t, h] = scale * (S.T @ q[n, t, h])
                prefix[n, t, h] = S
    return y, e, prefix


def mtp_commit(k, alpha, beta, e, accepted, state):
    """Advance the live states by the accepted prefix of a verified block.

    Shapes: k [N, K, H, d_k]; alpha, beta [N, K, H]; e [N, K, H, d_v] (the
    misses mtp_verify returned); accepted [N] integers in 0 .. K;
    state [N, H, d_k, d_v].  Returns the new states (float64); ``state`` is
    not modified.
    """
    k, alpha, beta, e = _f64(k), _f64(alpha), _f64(beta), _f64(e)
    S = _f64(state).copy()
    N, K, H, _ = k.shape
    for n in range(N):
        j = int(accepted[n])
        if not 0 <= j <= K:
            raise ValueError(f"accepted[{n}] = {j} outside 0..{K}")
        for h in range(H):
            for t in range(j):
                S[n, h] = alpha[n, t, h] * S[n, h] + beta[n, t, h] * np.outer(k[n, t, h], e[n, t, h])
    return S
