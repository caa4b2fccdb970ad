"""Plain float64 definition of the QSA (Qwen Sparse Attention) indexer.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
calls into this file, and this file never calls the HIP library.

Source: "On the Design of Qwen3.8-Next Architecture", slinene ai-papers-daily
page, Module B (Qwen Sparse Attention): a compressed MQA indexer with H query
heads and one shared key head.  Per sequence of n tokens, with block size r:
  * queries:  q_i^h = PRoPE(RMSNorm(q_proj_i^h), i)
  * keys are mean-pooled over non-overlapping blocks of r tokens first, then
    normalised, and only then rotated, at the block's start position p_b = b r:
        kbar_b = PRoPE(RMSNorm(mean(k_{p_b} .. k_{p_b + r - 1})), p_b),  b < floor(n / r)
    (the page stresses that pooling comes before the rotary embedding);
  * block-causal scores over complete blocks only:
        I_ib = sum_h ReLU(<q_i^h, kbar_b>)   if p_b + r - 1 <= i,  else -inf
  * selection: K_B = ceil(K / r) blocks per query, the K_B best complete blocks;
    the attended tokens are those blocks expanded, cut to the budget K, plus the
    tail tokens r floor((i + 1) / r) .. i of the current incomplete block.
The same selection is described on the rainbus digest (method step (2)).

Readings where the pages leave a step open:
  * the partial rotary embedding acts on the first ``rope_dims`` (64) of the
    head's 128 dimensions, in rotate-half pairs (j, j + rope_dims / 2) with
    angle pos * base^(-2 j / rope_dims), base 10000;
  * RMSNorm(x) = x / sqrt(mean(x^2) + eps) * w with eps = 1e-6 and w = 1 unless
    a weight is given;
  * when fewer than K_B complete blocks exist, all of them are selected;
  * ties in the score are broken towards the later block (larger b), so the
    selected set is unique; the block indices are reported in ascending order,
    padded with -1 up to K_B.

Parity pins live in tests/test_oracle_qsa.py.
"""

import math

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def rmsnorm(x, eps=1e-6, weight=None):
    """x / sqrt(mean(x^2) + eps) over the last axis, times ``weight`` if given."""
    x = _f64(x)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return y if weight is None else y * _f64(weight)


def partial_rope(x, pos, rope_dims=64, base=10000.0):
    """Rotate the first ``rope_dims`` entries of the last axis in rotate-half
    pairs (j, j + rope_dims / 2) by pos * base^(-2 j / rope_dims).

    x [..., D]; pos broadcastable to x.shape[:-1].
    """
    x = _f64(x).copy()
    half = rope_dims // 2
    if half == 0:
        return x
    j = np.arange(half, dtype=np.float64)
    ang = _f64(pos)[..., None] * base ** (-2.0 * j / rope_dims)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half].copy(), x[..., half:rope_dims].copy()
    x[..., :half] = a * c - b * s
    x[..., half:rope_dims] = b * c + a * s
    return x


def qsa_prep(q_proj, k_proj, r=4, rope_dims=64, base=10000.0, eps=1e-6, q_weight=None, k_weight=None):
    """Indexer operands from the projected streams.

    q_proj [B, n, H, D]; k_proj [B, n, D].  Returns (q [B, n, H, D],
    kbar [B, n // r, D]) in float64.
    """
    q_proj, k_proj = _f64(q_proj), _f64(k_proj)
    B, n, H, D = q_proj.shape
    pos = np.arange(n, dtype=np.float64)
    q = partial_rope(rmsnorm(q_proj, eps, q_weight), pos[None, :, None], rope_dims, base)
    nb = n // r
    pooled = k_proj[:, :nb * r].reshape(B, nb, r, D).mean(axis=2)
    kbar = partial_rope(rmsnorm(pooled, eps, k_weight), (np.arange(nb) * r)[None, :], rope_dims, base)
    return q, kbar


def qsa_scores(q, kbar, r=4):
    """I [B, n, nb] = sum_h ReLU(<q_i^h, kbar_b>) on complete past blocks, -inf elsewhere."""
    q, kbar = _f64(q), _f64(kbar)
    B, n, H, D = q.shape
    nb = kbar.shape[1]
    dots = np.einsum("bihd,bjd->bihj", q, kbar)                  # [B, n, H, nb]
    I = np.maximum(dots, 0.0).sum(axis=2)
    i = np.arange(n)[:, None]
    b = np.arange(nb)[None, :]
    complete = b * r + r - 1 <= i
    return np.where(complete[None], I, -np.inf)


def qsa_select(q, kbar, r=4, K=2048):
    """Selected block indices [B, n, K_B] (int64, ascending, -1 padded), K_B = ceil(K / r).

    For query i the candidates are the complete blocks b < floor((i + 1) / r);
    they are ranked by score, larger first, and among equal scores by block
    index, larger first; the first min(K_B, #candidates) are selected.
    """
    KB = -(-K // r)
    I = qsa_scores(q, kbar, r)
    B, n, nb = I.shape
    out = np.full((B, n, KB), -1, dtype=np.int64)
    for bb in range(B):
        for i in range(n):
            m = (i + 1) // r
            if m == 0:
                continue
            cand = np.arange(m)
            # lexsort: last key is primary -> sort by (-score, -index)
            order = np.lexsort((-cand, -I[bb, i, :m]))
            chosen = np.sort(cand[order[:min(KB, m)]])
            out[bb, i, :len(chosen)] = chosen
    return out


def qsa_token_set(blocks, i, r=4, K=2048):
    """Tokens attended by query i: its selected blocks expanded to tokens and
    cut to the budget K, plus the tail r floor((i + 1) / r) .. i."""
    toks = []
    for b in blocks:
        if b < 0:
            continue
        toks.extend(range(b * r, b * r + r))
    toks = toks[:K]
    tail = list(range(r * ((i + 1) // r), i + 1))
    return sorted(set(toks) | set(tail))
