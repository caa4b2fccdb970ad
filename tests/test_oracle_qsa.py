"""Pins of the float64 QSA indexer oracle (oracle/qsa_ref.py): a hand-worked
example, properties of the rotary embedding and of RMSNorm, the pool-then-rotate
ordering the pages insist on, block causality, top-K against a brute-force
subset search, the tie rule, and planted mistakes.  CPU only."""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import partial_rope, qsa_prep, qsa_scores, qsa_select, qsa_token_set, rmsnorm

HERE = os.path.dirname(os.path.abspath(__file__))
FIX = json.load(open(os.path.join(HERE, "golden", "qsa_example.json")))


def _fixture_inputs():
    q = np.array(FIX["q_proj"], dtype=np.float64)[None]        # [1, 6, 2, 2]
    k = np.array(FIX["k_proj"], dtype=np.float64)[None]        # [1, 6, 2]
    return q, k


def test_hand_example_prep_and_scores():
    q, k = _fixture_inputs()
    qq, kbar = qsa_prep(q, k, r=2, rope_dims=0, eps=0.0)
    np.testing.assert_array_equal(qq, q)
    np.testing.assert_array_equal(kbar[0], np.array(FIX["kbar"], dtype=np.float64))
    I = qsa_scores(qq, kbar, r=2)[0]
    expect = np.array([[(-np.inf if v is None else v) for v in row] for row in FIX["scores"]])
    np.testing.assert_array_equal(I, expect)


@pytest.mark.parametrize("K,key", [(2, "select_K2"), (4, "select_K4")])
def test_hand_example_selection(K, key):
    q, k = _fixture_inputs()
    qq, kbar = qsa_prep(q, k, r=2, rope_dims=0, eps=0.0)
    np.testing.assert_array_equal(qsa_select(qq, kbar, r=2, K=K)[0], np.array(FIX[key]))


def test_hand_example_token_sets():
    for i, toks in FIX["token_sets_K2"].items():
        blocks = np.array(FIX["select_K2"][int(i)])
        assert qsa_token_set(blocks, int(i), r=2, K=2) == toks


def test_rope_hand_value():
    x = np.array(FIX["rope"]["x"], dtype=np.float64)
    np.testing.assert_allclose(partial_rope(x, 1.0, rope_dims=4), FIX["rope"]["expected"], rtol=0, atol=1e-15)


def test_rope_is_a_rotation_with_relative_angles():
    """Norm preserved; <R(x, m), R(y, n)> on the rotary part depends on m - n only;
    dimensions past rope_dims are untouched."""
    rng = np.random.default_rng(1)
    x, y = rng.standard_normal(128), rng.standard_normal(128)
    for m, n in [(0, 0), (5, 3), (1000, 7)]:
        a, b = partial_rope(x, m), partial_rope(y, n)
        np.testing.assert_allclose(np.linalg.norm(a), np.linalg.norm(x), rtol=1e-14)
        np.testing.assert_array_equal(a[64:], x[64:])
        a2, b2 = partial_rope(x, m + 11), partial_rope(y, n + 11)
        np.testing.assert_allclose(a[:64] @ b[:64], a2[:64] @ b2[:64], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(partial_rope(x, 0), x)


def test_rmsnorm_unit_rms_and_weight():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 128)) * 3.0
    y = rmsnorm(x, eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    w = rng.standard_normal(128)
    np.testing.assert_allclose(rmsnorm(x, 0.0, w), y * w, rtol=1e-14)


def _rand(seed, B=2, n=37, H=4, D=16):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, n, H, D)), rng.standard_normal((B, n, D))


def test_pooling_comes_before_rotation():
    """The pooled key is the rotation of the pooled normalised mean, not the
    mean of rotated keys (the ordering point of the slinene page)."""
    q, k = _rand(3, n=16)
    _, kbar = qsa_prep(q, k, r=4, rope_dims=8)
    pooled = k[:, :16].reshape(2, 4, 4, 16).mean(axis=2)
    expect = partial_rope(rmsnorm(pooled), (np.arange(4) * 4)[None, :], rope_dims=8)
    np.testing.assert_allclose(kbar, expect, rtol=0, atol=1e-14)
    rotated_first = partial_rope(k, np.arange(16)[None, :], rope_dims=8)
    wrong = partial_rope(rmsnorm(rotated_first.reshape(2, 4, 4, 16).mean(axis=2)), 0.0, rope_dims=0)
    assert np.max(np.abs(wrong - kbar)) > 1e-2


def test_block_causality():
    """Query i scores exactly the blocks b with b r + r - 1 <= i; the current
    incomplete block is never scored; a later query never changes earlier rows."""
    q, k = _rand(4, n=23)
    qq, kbar = qsa_prep(q, k, r=4, rope_dims=8)
    I = qsa_scores(qq, kbar, r=4)
    for i in range(23):
        finite = np.isfinite(I[0, i])
        assert finite.sum() == (i + 1) // 4
        assert np.all(finite[:(i + 1) // 4])
    q2, k2 = q.copy(), k.copy()
    q2[:, 15:] += 1.0
    k2[:, 16:] -= 2.0
    qq2, kbar2 = qsa_prep(q2, k2, r=4, rope_dims=8)
    np.testing.assert_array_equal(qsa_select(qq2, kbar2, r=4, K=8)[:, :15], qsa_select(qq, kbar, r=4, K=8)[:, :15])


def test_topk_equals_best_subset_brute_force():
    """With continuous scores (no ties) the selected set is the subset of size
    min(K_B, m) with the largest score sum, found by trying every subset."""
    q, k = _rand(5, B=1, n=29, H=4, D=8)
    qq, kbar = qsa_prep(q, k, r=3, rope_dims=4)
    I = qsa_scores(qq, kbar, r=3)
    sel = qsa_select(qq, kbar, r=3, K=8)                            # K_B = 3
    for i in range(29):
        m = (i + 1) // 3
        if m == 0:
            assert np.all(sel[0, i] == -1)
            continue
        size = min(3, m)
        best = max(itertools.combinations(range(m), size), key=lambda s: sum(I[0, i, list(s)]))
        np.testing.assert_array_equal(sel[0, i, :size], sorted(best))
        assert np.all(sel[0, i, size:] == -1)


def test_ties_go_to_the_later_block():
    """All-zero scores (every head negative): the latest K_B complete blocks win."""
    q = -np.ones((1, 20, 2, 4))
    k = np.ones((1, 20, 4))
    qq, kbar = qsa_prep(q, k, r=2, rope_dims=0)
    sel = qsa_select(qq, kbar, r=2, K=4)                             # K_B = 2
    for i in range(20):
        m = (i + 1) // 2
        expect = [b for b in range(max(0, m - 2), m)]
        np.testing.assert_array_equal(sel[0, i, :len(expect)], expect)


def test_budget_larger_than_history_selects_every_complete_block():
    q, k = _rand(6, n=20)
    qq, kbar = qsa_prep(q, k, r=4, rope_dims=8)
    sel = qsa_select(qq, kbar, r=4, K=2048)
    for i in range(20):
        m = (i + 1) // 4
        np.testing.assert_array_equal(sel[0, i, :m], np.arange(m))
        assert np.all(sel[0, i, m:] == -1)


def _mutant_scores(mistake):
    def scores(q, kbar, r):
        B, n, H, D = q.shape
        nb = kbar.shape[1]
        dots = np.einsum("bihd,bjd->bihj", q, kbar)
        I = np.maximum(dots.sum(axis=2), 0.0) if mistake == "relu_after_head_sum" else np.maximum(dots, 0.0).sum(axis=2)
        i = np.arange(n)[:, None]
        b = np.arange(nb)[None, :]
        complete = (b * r <= i) if mistake == "incomplete_block_scored" else (b * r + r - 1 <= i)
        return np.where(complete[None], I, -np.inf)
    return scores


@pytest.mark.parametrize("mistake", ["relu_after_head_sum", "incomplete_block_scored"])
def test_hand_example_catches_planted_score_mistakes(mistake):
    q, k = _fixture_inputs()
    qq, kbar = qsa_prep(q, k, r=2, rope_dims=0, eps=0.0)
    got = _mutant_scores(mistake)(qq, kbar, 2)[0]
    expect = np.array([[(-np.inf if v is None else v) for v in row] for row in FIX["scores"]])
    assert not np.array_equal(got, expect)
