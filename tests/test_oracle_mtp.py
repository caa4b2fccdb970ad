"""Pins of the float64 multi-token decode oracle (oracle/mtp_ref.py).

The verify step is a K-token run of the recurrence from a live state, so every
recurrence pin (compact form, pure decay, exact retrieval, LMS step, scalar
closed form, brute-force unrolling, linearity, causality, segment composition)
and the hand-worked four-token example apply to it directly.  The commit step
is pinned by what rollback must give: the state after exactly the accepted
prefix, identical to a plain run over that prefix.  CPU only."""

import json
import os

import numpy as np
import pytest

from oracle import gated_delta_recurrence, mtp_commit, mtp_verify
from tests import oracle_pins

HERE = os.path.dirname(os.path.abspath(__file__))
FIXTURE = json.load(open(os.path.join(HERE, "golden", "hand_example.json")))


def _as_recurrence(verify):
    """mtp_verify seen as impl(q, k, v, alpha, beta, initial_state, scale) -> (y, S_T)."""
    def impl(q, k, v, alpha, beta, initial_state=None, scale=1.0):
        q = np.asarray(q, np.float64)
        B, T, H, dk = q.shape
        dv = np.asarray(v).shape[-1]
        S0 = np.zeros((B, H, dk, dv)) if initial_state is None else initial_state
        y, _, prefix = verify(q, k, v, alpha, beta, S0, scale=scale)
        return y, (prefix[:, -1] if T else np.array(S0, np.float64))
    return impl


@pytest.mark.parametrize("pin", oracle_pins.RECURRENCE_PINS, ids=lambda p: p.__name__)
def test_verify_meets_recurrence_pin(pin):
    assert pin(_as_recurrence(mtp_verify)) < 1e-9


def test_verify_hand_example():
    assert oracle_pins.pin_hand_example(_as_recurrence(mtp_verify), FIXTURE) < 1e-12


def _draft_block(seed, N=3, K=4, H=2, dk=6, dv=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, K, H, dk))
    k = rng.standard_normal((N, K, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, K, H, dv))
    a = rng.uniform(0.2, 0.99, (N, K, H))
    b = rng.uniform(0.05, 0.95, (N, K, H))
    S0 = rng.standard_normal((N, H, dk, dv))
    return q, k, v, a, b, S0


def test_prefix_states_are_the_recurrence_states():
    """Prefix state t equals the final state of an independent t-token run."""
    q, k, v, a, b, S0 = _draft_block(1)
    y, e, prefix = mtp_verify(q, k, v, a, b, S0, scale=0.7)
    for t in range(1, q.shape[1] + 1):
        y_r, S_r = gated_delta_recurrence(q[:, :t], k[:, :t], v[:, :t], a[:, :t], b[:, :t], S0, scale=0.7)
        np.testing.assert_allclose(prefix[:, t - 1], S_r, rtol=0, atol=1e-12)
        np.testing.assert_allclose(y[:, :t], y_r, rtol=0, atol=1e-12)


def test_miss_is_the_decayed_state_error():
    """e_t = v_t - alpha_t S_{t-1}^T k_t with S_{t-1} the previous prefix state."""
    q, k, v, a, b, S0 = _draft_block(2)
    _, e, prefix = mtp_verify(q, k, v, a, b, S0)
    N, K, H, _ = k.shape
    for n in range(N):
        for h in range(H):
            S_prev = S0[n, h]
            for t in range(K):
                expect = v[n, t, h] - a[n, t, h] * (k[n, t, h] @ S_prev)
                np.testing.assert_allclose(e[n, t, h], expect, rtol=0, atol=1e-12)
                S_prev = prefix[n, t, h]


def test_verify_leaves_the_state_alone():
    q, k, v, a, b, S0 = _draft_block(3)
    before = S0.copy()
    mtp_verify(q, k, v, a, b, S0)
    np.testing.assert_array_equal(S0, before)


@pytest.mark.parametrize("accepted", [[0, 0, 0], [4, 4, 4], [1, 2, 3], [3, 0, 4]])
def test_commit_gives_the_accepted_prefix_state(accepted):
    """Rollback: committing j accepted drafts lands on the j-token run's state."""
    q, k, v, a, b, S0 = _draft_block(4)
    _, e, prefix = mtp_verify(q, k, v, a, b, S0)
    S = mtp_commit(k, a, b, e, np.array(accepted), S0)
    for n, j in enumerate(accepted):
        if j == 0:
            np.testing.assert_array_equal(S[n], S0[n])
        else:
            _, S_r = gated_delta_recurrence(q[n:n + 1, :j], k[n:n + 1, :j], v[n:n + 1, :j],
                                            a[n:n + 1, :j], b[n:n + 1, :j], S0[n:n + 1])
            np.testing.assert_allclose(S[n], S_r[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(S[n], prefix[n, j - 1], rtol=0, atol=1e-12)


def test_commit_then_verify_rest_matches_one_block():
    """Accept j drafts, then verify the rest from the committed state: the
    outputs of the remaining tokens equal those of the original block."""
    q, k, v, a, b, S0 = _draft_block(5, K=6)
    y, e, _ = mtp_verify(q, k, v, a, b, S0)
    j = 2
    S = mtp_commit(k, a, b, e, np.full(q.shape[0], j), S0)
    y2, _, _ = mtp_verify(q[:, j:], k[:, j:], v[:, j:], a[:, j:], b[:, j:], S)
    np.testing.assert_allclose(y2, y[:, j:], rtol=0, atol=1e-12)


def test_commit_exact_retrieval_after_accepting_orthonormal_keys():
    """alpha = beta = 1, orthonormal keys, zero state: after accepting j drafts
    the state returns v_i for each accepted key k_i and nothing for the rest
    (the targeted erase-write of the rainbus digest's prerequisites)."""
    rng = np.random.default_rng(6)
    K, dk, dv = 5, 8, 3
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = basis[:K][None, :, None]                       # [1, K, 1, dk]
    q = k.copy()
    v = rng.standard_normal((1, K, 1, dv))
    ones = np.ones((1, K, 1))
    S0 = np.zeros((1, 1, dk, dv))
    _, e, _ = mtp_verify(q, k, v, ones, ones, S0)
    for j in range(K + 1):
        S = mtp_commit(k, ones, ones, e, np.array([j]), S0)[0, 0]
        for i in range(K):
            expect = v[0, i, 0] if i < j else np.zeros(dv)
            np.testing.assert_allclose(k[0, i, 0] @ S, expect, rtol=0, atol=1e-12)


def test_pure_decay_closed_form():
    """beta = 0: nothing is written; prefix t = (prod of alphas) S0 and the miss
    is v_t minus the decayed state's recall."""
    q, k, v, a, _, S0 = _draft_block(7)
    zero = np.zeros_like(a)
    y, e, prefix = mtp_verify(q, k, v, a, zero, S0)
    G = np.cumprod(a, axis=1)                          # [N, K, H]
    np.testing.assert_allclose(prefix, G[..., None, None] * S0[:, None], rtol=0, atol=1e-12)
    recall = np.einsum("nthk,nhkv->nthv", k, S0)
    np.testing.assert_allclose(e, v - G[..., None] * recall, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y, G[..., None] * np.einsum("nthk,nhkv->nthv", q, S0), rtol=0, atol=1e-12)


def test_commit_rejects_out_of_range_counts():
    q, k, v, a, b, S0 = _draft_block(8)
    _, e, _ = mtp_verify(q, k, v, a, b, S0)
    with pytest.raises(ValueError):
        mtp_commit(k, a, b, e, np.array([0, 5, 1]), S0)
    with pytest.raises(ValueError):
        mtp_commit(k, a, b, e, np.array([0, -1, 1]), S0)


def _commit_mutant(mistake):
    def commit(k, alpha, beta, e, accepted, state):
        S = np.array(state, np.float64)
        N, K, H, _ = k.shape
        for n in range(N):
            j = int(accepted[n])
            if mistake == "off_by_one":
                j = min(j + 1, K)
            for h in range(H):
                for t in range(j):
                    a = alpha[n, t, h] if mistake != "decay_index_shift" else alpha[n, max(t - 1, 0), h]
                    w = beta[n, t, h] if mistake != "dropped_beta" else 1.0
                    if mistake == "write_before_decay":
                        S[n, h] = a * (S[n, h] + w * np.outer(k[n, t, h], e[n, t, h]))
                    else:
                        S[n, h] = a * S[n, h] + w * np.outer(k[n, t, h], e[n, t, h])
        return S
    return commit


@pytest.mark.parametrize("mistake", [None, "off_by_one", "decay_index_shift", "dropped_beta",
                                     "write_before_decay"])
def test_commit_pins_catch_planted_mistakes(mistake):
    """The prefix-state pin catches each plausible commit mistake."""
    q, k, v, a, b, S0 = _draft_block(9)
    _, e, prefix = mtp_verify(q, k, v, a, b, S0)
    accepted = np.array([2, 3, 1])
    S = _commit_mutant(mistake)(k, a, b, e, accepted, S0)
    dev = max(np.max(np.abs(S[n] - prefix[n, j - 1])) for n, j in enumerate(accepted))
    if mistake is None:
        assert dev < 1e-12
    else:
        assert dev > 1e-6
