"""gdn_qsa_prep / gdn_qsa_select on the GPU against the float64 QSA indexer
oracle (oracle/qsa_ref.py)."""

import numpy as np
import pytest
import torch

from oracle import qsa_prep, qsa_scores, qsa_select
from tests.gpu_util import dev, host, say
from workloads import qsa_inputs, qsa_select_inputs
import linear_attention_recurrence_rule_amd as gdn

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _check_prep(got, ref, dtype, name):
    """fp32: float32 rounding of unit-scale values; bf16: one bf16 rounding of
    the exact value (half an ulp, 2^-9 relative) plus the float32 error of the
    value before rounding, which can push it over a rounding midpoint."""
    err = np.abs(got - ref)
    if dtype == "f32":
        bound = 2e-6 * (1.0 + np.abs(ref))
    else:
        bound = (2.0 ** -8 + 1e-5) * np.abs(ref) + 1e-6
    worst = float(np.max(err - bound))
    say(f"    {name}: max|d| = {float(np.max(err)):.3e}, worst margin {worst:.3e}")
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), f"{name}: {int(np.sum(err > bound))} entries over the bound"


@pytest.mark.parametrize("D,R", [(32, 32), (64, 64), (128, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prep(D, R, dtype):
    say(f"qsa prep D={D} R={R} {dtype}")
    B, n, H, r = 2, 203, 4, 4
    d = qsa_inputs(B, n, H, D, dtype, seed=D)
    rng = np.random.default_rng(D + 1)
    qw = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    kw = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    q, kbar = gdn.gdn_qsa_prep(dev(d["q_proj"], dtype), dev(d["k_proj"], dtype), r=r, rope_dims=R,
                               q_weight=dev(qw), k_weight=dev(kw))
    q_ref, k_ref = qsa_prep(d["q_proj"], d["k_proj"], r=r, rope_dims=R, q_weight=qw, k_weight=kw)
    _check_prep(host(q), q_ref, dtype, "q")
    _check_prep(host(kbar), k_ref, dtype, "kbar")


def test_prep_long_positions():
    """65536 tokens: the rotation phase at large positions (checked on every row)."""
    say("qsa prep n=65536")
    d = qsa_inputs(1, 65536, 4, 128, "bf16", seed=3)
    q, kbar = gdn.gdn_qsa_prep(dev(d["q_proj"], "bf16"), dev(d["k_proj"], "bf16"))
    q_ref, k_ref = qsa_prep(d["q_proj"], d["k_proj"])
    _check_prep(host(q), q_ref, "bf16", "q")
    _check_prep(host(kbar), k_ref, "bf16", "kbar")


def _row_scores(q, kbar, i, r):
    """Oracle scores of query i's candidate blocks and, per block, the fp32
    error bound of the GPU's sum (D + H + 2 roundings of the absolute terms)."""
    m = (i + 1) // r
    qi = q[i].astype(np.float64)                      # [H, D]
    kb = kbar[:m].astype(np.float64)                  # [m, D]
    dots = qi @ kb.T                                  # [H, m]
    I = np.maximum(dots, 0.0).sum(axis=0)
    absum = (np.abs(qi) @ np.abs(kb).T).sum(axis=0)
    eps = (qi.shape[1] + qi.shape[0] + 2) * U32 * absum
    return I, eps


def _oracle_row_select(I, KB):
    m = len(I)
    cand = np.arange(m)
    order = np.lexsort((-cand, -I))
    return np.sort(cand[order[:min(KB, m)]])


def _check_rows(got, q, kbar, rows, r, KB, name):
    """Exact agreement with the oracle, except on rows whose selection boundary
    lies within the float32 error of the scores: there the GPU's set must still
    be a valid top-K_B of the oracle scores up to that error."""
    near = 0
    for i in rows:
        I, eps = _row_scores(q, kbar, i, r)
        m = len(I)
        g = got[i]
        size = min(KB, m)
        assert np.all(g[size:] == -1), f"{name} row {i}: padding"
        sel = g[:size]
        assert np.all(np.diff(sel) > 0) and (size == 0 or (sel[0] >= 0 and sel[-1] < m)), f"{name} row {i}: order"
        ref = _oracle_row_select(I, KB)
        if np.array_equal(sel, ref):
            continue
        near += 1
        rest = np.setdiff1d(np.arange(m), sel)
        assert (I[sel] + eps[sel]).min() >= (I[rest] - eps[rest]).max(), \
            f"{name} row {i}: not a top-{KB} set within the fp32 error"
    say(f"    {name}: {len(rows)} rows checked, {near} differ from the oracle within the fp32 error")
    assert near <= max(1, len(rows) // 100)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n,K", [(63, 16), (200, 16), (1000, 64), (1000, 2048), (1024, 256)])
@pytest.mark.parametrize("D", [32, 128])
def test_select(dtype, n, K, D):
    say(f"qsa select n={n} K={K} D={D} {dtype}")
    B, H, r = 2, 4, 4
    d = qsa_select_inputs(B, n, r, H, D, dtype, seed=n + K + D)
    idx = host(gdn.gdn_qsa_select(dev(d["q"], dtype), dev(d["kbar"], dtype), r=r, K=K)).astype(np.int64)
    KB = -(-K // r)
    ref = qsa_select(d["q"], d["kbar"], r=r, K=K)
    assert idx.shape == ref.shape
    for b in range(B):
        _check_rows(idx[b], d["q"][b], d["kbar"][b], range(n), r, KB, f"batch {b}")


def test_select_all_zero_scores_take_the_latest_blocks():
    """Every head negative against every block: all scores are exactly 0 and the
    tie rule picks the latest K_B complete blocks."""
    say("qsa select all-zero scores")
    B, n, H, D, r, K = 1, 300, 4, 64, 4, 32
    rng = np.random.default_rng(8)
    x = np.abs(rng.standard_normal((B, n // r, D))).astype(np.float32) + 0.1
    q = -np.abs(rng.standard_normal((B, n, H, D))).astype(np.float32) - 0.1
    idx = host(gdn.gdn_qsa_select(dev(q, "bf16"), dev(x, "bf16"), r=r, K=K)).astype(np.int64)
    KB = K // r
    for i in range(n):
        m = (i + 1) // r
        expect = np.arange(max(0, m - KB), m)
        np.testing.assert_array_equal(idx[0, i, :len(expect)], expect)
        assert np.all(idx[0, i, len(expect):] == -1)


def test_select_long_context_sampled_rows():
    """65536 tokens (16384 blocks), H = 4, D = 128, K = 2048 (512 blocks): one
    launch, 96 sampled query rows (the latest ones have 16384 candidates)."""
    say("qsa select n=65536")
    n, r, K = 65536, 4, 2048
    d = qsa_select_inputs(1, n, r, 4, 128, "bf16", seed=11)
    idx = host(gdn.gdn_qsa_select(dev(d["q"], "bf16"), dev(d["kbar"], "bf16"), r=r, K=K)).astype(np.int64)
    rng = np.random.default_rng(12)
    rows = sorted(set(rng.integers(0, n, 80).tolist()) | {2047, 2048, 2051, 4095, n - 4, n - 3, n - 2, n - 1}
                  | set(range(n - 8, n)))
    _check_rows(idx[0], d["q"][0], d["kbar"][0], rows, r, K // r, "sampled")


def test_select_rows_longer_than_one_bitmap_chunk():
    """40000 tokens at r = 2 (20000 blocks): the latest rows have more
    candidate blocks than one 16384-block bitmap chunk of the merge, so their
    ascending output is assembled chunk by chunk."""
    say("qsa select n=40000 r=2")
    n, r, K = 40000, 2, 1024
    d = qsa_select_inputs(1, n, r, 4, 128, "bf16", seed=31)
    idx = host(gdn.gdn_qsa_select(dev(d["q"], "bf16"), dev(d["kbar"], "bf16"), r=r, K=K)).astype(np.int64)
    rng = np.random.default_rng(32)
    rows = sorted(set(rng.integers(2 * 16384, n, 16).tolist()) | {2 * 16384 - 1, 2 * 16384, n - 2, n - 1})
    _check_rows(idx[0], d["q"][0], d["kbar"][0], rows, r, K // r, "beyond one chunk")


@pytest.mark.parametrize("H", [1, 3])
def test_select_other_head_counts(H):
    """Head counts other than four take the stored-score path."""
    say(f"qsa select H={H}")
    B, n, D, r, K = 2, 700, 64, 4, 64
    d = qsa_select_inputs(B, n, r, H, D, "bf16", seed=H + 40)
    idx = host(gdn.gdn_qsa_select(dev(d["q"], "bf16"), dev(d["kbar"], "bf16"), r=r, K=K)).astype(np.int64)
    for b in range(B):
        _check_rows(idx[b], d["q"][b], d["kbar"][b], range(n), r, K // r, f"batch {b}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_select_equal_scores_take_the_latest_blocks(dtype):
    """Every block has the same key, so every score of a query is the same
    positive number: the tie rule picks the latest K_B blocks.  Queries with
    more than 1024 such candidates take the exact recomputation pass."""
    say(f"qsa select equal scores {dtype}")
    B, n, H, D, r, K = 1, 4800, 4, 64, 4, 64
    rng = np.random.default_rng(17)
    x = (np.abs(rng.standard_normal(D)) + 0.1).astype(np.float32)
    kbar = np.broadcast_to(x, (B, n // r, D)).copy()
    q = (np.abs(rng.standard_normal((B, n, H, D))) + 0.1).astype(np.float32)
    idx = host(gdn.gdn_qsa_select(dev(q, dtype), dev(kbar, dtype), r=r, K=K)).astype(np.int64)
    KB = K // r
    for i in range(n):
        m = (i + 1) // r
        expect = np.arange(max(0, m - KB), m)
        np.testing.assert_array_equal(idx[0, i, :len(expect)], expect, err_msg=f"row {i}")
        assert np.all(idx[0, i, len(expect):] == -1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_select_threshold_below_the_histogram_window(dtype):
    """Block 0's key is 10^6 times longer than the others, which puts the other
    scores some 20 octaves below the queries' bound, under the 15.9-octave
    histogram window: the threshold lies in the underflow bin and is ranked
    exactly by the merge (up to 1024 candidates) or by the exact recomputation
    pass (more)."""
    say(f"qsa select huge key {dtype}")
    B, n, H, D, r, K = 1, 6000, 4, 64, 4, 256
    d = qsa_select_inputs(B, n, r, H, D, dtype, seed=23)
    kbar = d["kbar"].copy()
    kbar[:, 0] *= 1e6
    if dtype == "bf16":
        kbar = host(dev(kbar, "bf16")).astype(np.float32)     # the exact values the GPU sees
    idx = host(gdn.gdn_qsa_select(dev(d["q"], dtype), dev(kbar, dtype), r=r, K=K)).astype(np.int64)
    rows = list(range(0, n, 7)) + list(range(n - 40, n))
    _check_rows(idx[0], d["q"][0], kbar[0], rows, r, K // r, "huge key")


def test_select_fewer_positive_scores_than_the_budget():
    """Most scores are exactly zero and a few blocks score positive: every
    positive block is selected and the latest zeros fill the budget."""
    say("qsa select few positives")
    B, n, H, D, r, K = 1, 300, 4, 64, 4, 32
    rng = np.random.default_rng(31)
    x = (np.abs(rng.standard_normal((B, n // r, D))) + 0.1).astype(np.float32)
    x[:, [3, 10, 20, 40, 60]] *= -1.0
    q = (-np.abs(rng.standard_normal((B, n, H, D))) - 0.1).astype(np.float32)
    idx = host(gdn.gdn_qsa_select(dev(q, "bf16"), dev(x, "bf16"), r=r, K=K)).astype(np.int64)
    qh = host(dev(q, "bf16")).astype(np.float32)
    xh = host(dev(x, "bf16")).astype(np.float32)
    ref = qsa_select(qh, xh, r=r, K=K)
    np.testing.assert_array_equal(idx, ref)
