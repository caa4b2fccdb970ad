"""Plain float64 definition of the GDN front end (projected streams -> q, k, v, alpha, beta).

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
calls into this file, and this file never calls the HIP library.

Source: "On the Design of Qwen3.8-Next Architecture", slinene ai-papers-daily
page, Module A (Gated DeltaNet), parameterisation block; the same structure is
drawn in the Gated DeltaNet figure of the paper.rainbus.top digest (Figure 2:
short causal convolutions on the query, key and value streams, L2
normalisation of queries and keys, decay and write gates).  Per token t and
head h, from the projected streams (the projections themselves are not part
of this step):
    q_t = L2Norm(SiLU(ShortConv(q_proj)_t))
    k_t = L2Norm(SiLU(ShortConv(k_proj)_t))
    v_t = SiLU(ShortConv(v_proj)_t)
    beta_t  = sigmoid(b_logit_t)
    alpha_t = exp(-exp(A_h) * softplus(a_logit_t + b_alpha_h))

Readings where the pages leave a step open:
  * ShortConv is a causal depthwise convolution over time, one filter of
    width W per channel and head, no bias:
        conv_t[c] = sum_{j=0}^{W-1} w[h, c, j] * x_{t-(W-1)+j}[c],
    with x_s = 0 before the sequence start unless the caller passes the W-1
    preceding rows (``*_history``).  The pages give no width.
  * L2Norm(x) = x / sqrt(sum(x^2) + eps) over the head dimension; the pages
    give no epsilon (``eps``, 1e-6 by default).
  * SiLU(x) = x * sigmoid(x).
  * A and b_alpha are per-head scalars.

Parity pins for this function live in tests/test_oracle_frontend.py.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def short_conv(x, w, history=None):
    """Causal depthwise convolution over time.

    x [B, T, H, d]; w [H, d, W]; history [B, W-1, H, d] or None (zeros).
    Returns conv [B, T, H, d] float64 with conv_t = sum_j w[..., j] x_{t-(W-1)+j}.
    """
    x, w = _f64(x), _f64(w)
    B, T, H, d = x.shape
    W = w.shape[-1]
    if history is None:
        history = np.zeros((B, W - 1, H, d))
    padded = np.concatenate([_f64(history), x], axis=1)      # [B, W-1+T, H, d]
    out = np.zeros((B, T, H, d))
    for j in range(W):
        out += w[None, None, :, :, j] * padded[:, j:j + T]
    return out


def silu(x):
    x = _f64(x)
    return x * _sigmoid(x)


def l2norm(x, eps=1e-6):
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gdn_frontend(q_proj, k_proj, v_proj, conv_q, conv_k, conv_v, a_logit, b_logit, A, b_alpha,
                 q_history=None, k_history=None, v_history=None, eps=1e-6):
    """q, k, v, alpha, beta of the mixer from its projected streams (float64).

    Shapes: q_proj, k_proj [B, T, H, d_k]; v_proj [B, T, H, d_v]; conv_* [H, d, W];
    a_logit, b_logit [B, T, H]; A, b_alpha [H]; *_history [B, W-1, H, d] or None.
    """
    q = l2norm(silu(short_conv(q_proj, conv_q, q_history)), eps)
    k = l2norm(silu(short_conv(k_proj, conv_k, k_history)), eps)
    v = silu(short_conv(v_proj, conv_v, v_history))
    beta = _sigmoid(_f64(b_logit))
    alpha = np.exp(-np.exp(_f64(A))[None, None, :] * _softplus(_f64(a_logit) + _f64(b_alpha)[None, None, :]))
    return q, k, v, alpha, beta
