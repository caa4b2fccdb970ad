"""Plain float64 definitions of the three operations of the GDN token mixer.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
calls into this file, and this file never calls the HIP library.

Sources (pages on "On the Design of Qwen3.8-Next Architecture"):
  * slinene ai-papers-daily page, Module A (Gated DeltaNet), the four-line
    delta form: the state decays by alpha_t, the decayed state is read with
    k_t, the miss e_t = v_t - (decayed state)^T k_t is written back with
    strength beta_t along k_t, and the output reads the *updated* state with
    q_t.  The state is d_k x d_v (transposed relative to the original GDN
    paper), so the read is S^T k.
  * same page, Module A parameterisation: the output is
    sigma(W_z x) * RMSNorm(y) with a sigmoid (not SiLU) gate, and the RMSNorm
    is the zero-centred kind (its weight is stored as an offset from one).
  * paper.rainbus.top digest, method step (1): the same recurrence written as
    alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T.

Readings where the pages leave a step open:
  * no 1/sqrt(d_k) on the query (the pages show none); ``scale`` defaults to 1;
  * RMSNorm is taken per (token, head) over d_v with an epsilon the caller
    gives (1e-6 by default, the pages state none), weight (1 + w) with w of
    shape [d_v]; the gate multiplies after the norm.

Parity pins for every function here live in tests/test_oracle_pins.py.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def gated_delta_recurrence(q, k, v, alpha, beta, initial_state=None, scale=1.0):
    """Run the gated delta rule token by token.

    Shapes: q, k [B, T, H, d_k]; v [B, T, H, d_v]; alpha, beta [B, T, H];
    initial_state [B, H, d_k, d_v] or None (zeros).
    Returns (y [B, T, H, d_v], final_state [B, H, d_k, d_v]), float64.

    Per (b, h) and t = 0 .. T-1 (Module A, delta form):
        S_dec = alpha_t * S                    decay the whole state
        e     = v_t - S_dec^T k_t              what the decayed state misses
        S     = S_dec + beta_t * k_t e^T       rank-one write of the miss
        y_t   = scale * S^T q_t                read with the updated state
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta = _f64(alpha), _f64(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if initial_state is None:
        S = np.zeros((B, H, dk, dv))
    else:
        S = _f64(initial_state).copy()
    y = np.empty((B, T, H, dv))
    for t in range(T):
        S_dec = alpha[:, t, :, None, None] * S
        k_t = k[:, t]                                      # [B, H, dk]
        recalled = np.matmul(k_t[:, :, None, :], S_dec)[:, :, 0, :]   # S_dec^T k_t
        e = v[:, t] - recalled                             # [B, H, dv]
        S = S_dec + beta[:, t, :, None, None] * (k_t[:, :, :, None] * e[:, :, None, :])
        y[:, t] = scale * np.matmul(q[:, t][:, :, None, :], S)[:, :, 0, :]
    return y, S


def gated_delta_decode_step(q, k, v, alpha, beta, state, scale=1.0):
    """One recurrence step for a batch of live states (the decode case).

    Shapes: q, k [N, H, d_k]; v [N, H, d_v]; alpha, beta [N, H];
    state [N, H, d_k, d_v].  Returns (y [N, H, d_v], new_state), float64;
    the input state is not modified.  Same step as gated_delta_recurrence.
    """
    y, S = gated_delta_recurrence(_f64(q)[:, None], _f64(k)[:, None], _f64(v)[:, None],
                                  _f64(alpha)[:, None], _f64(beta)[:, None],
                                  initial_state=state, scale=scale)
    return y[:, 0], S


def gated_rmsnorm(y, z, weight=None, eps=1e-6):
    """Output epilogue sigma(z) * RMSNorm(y) with a zero-centred weight.

    Shapes: y, z [..., d_v]; weight [d_v] or None (all zero, i.e. the plain
    norm).  Per row over the last axis:
        o = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + weight)
    """
    y, z = _f64(y), _f64(z)
    w = np.zeros(y.shape[-1]) if weight is None else _f64(weight)
    mean_sq = np.mean(y * y, axis=-1, keepdims=True)
    normed = y / np.sqrt(mean_sq + eps)
    with np.errstate(over="ignore"):
        gate = 1.0 / (1.0 + np.exp(-z))
    return gate * normed * (1.0 + w)


def rel_err(x, ref):
    """max |x - ref| divided by the root-mean-square of ref (whole tensor)."""
    x, ref = _f64(x), _f64(ref)
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0.0:
        return float(np.max(np.abs(x - ref))) if x.size else 0.0
    return float(np.max(np.abs(x - ref)) / rms) if x.size else 0.0
