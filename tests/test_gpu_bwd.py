"""gdn_prefill_bwd on the GPU against the float64 backward oracle
(oracle/bwd_ref.py): every gradient, element by element, as max|d|/rms."""

import numpy as np
import pytest
import torch

from oracle import gated_delta_backward
from tests import oracle_pool
from tests.gpu_util import TOL, check, dev, host, say
from workloads import config_prefill_inputs, prefill_inputs
import linear_attention_recurrence_rule_amd as gdn

pytestmark = pytest.mark.gpu

# For fp32 inputs every contraction of the backward is float32 MFMA, with
# float32 chunk matrices and states in between (the float32 bound, 1e-4); for
# bf16 inputs the contractions take fp16 operands with float32 accumulation
# (the bf16 bound, 2e-2).
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "d_initial_state")


def _run(d, dtype, dy, S0=None, dST=None, scale=1.0):
    q, k, v = (dev(d[x], dtype) for x in ("q", "k", "v"))
    a, b = dev(d["alpha"]), dev(d["beta"])
    out = gdn.gdn_prefill_bwd(q, k, v, a, b, dev(dy), None if S0 is None else dev(S0),
                              None if dST is None else dev(dST), scale=scale)
    return [host(x) for x in out]


def _compare(got, ref, tol, heads=None):
    for name, g, r in zip(NAMES, got, ref):
        if heads is not None:
            g = g[:, :, heads] if g.ndim >= 3 and name != "d_initial_state" else g[:, heads]
        check(name, g, r, tol)


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 64, 150])
def test_bwd_small(D, dtype, T):
    say(f"bwd D={D} {dtype} T={T}")
    B, H = 2, 3
    d = prefill_inputs(B, T, H, D, D, dtype, -1.0, 0.5, seed=D + T, state_std=0.1)
    rng = np.random.default_rng([D, T, 5])
    dy = rng.standard_normal((B, T, H, D)).astype(np.float32)
    dST = rng.standard_normal((B, H, D, D)).astype(np.float32)
    got = _run(d, dtype, dy, d["initial_state"], dST, scale=0.8)
    ref = gated_delta_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dy, d["initial_state"], dST,
                               scale=0.8)
    _compare(got, ref, TOL[dtype])


def test_bwd_without_states():
    """No initial state and no final-state gradient (both read as zero)."""
    say("bwd without states")
    B, T, H, D = 1, 200, 2, 64
    d = prefill_inputs(B, T, H, D, D, "bf16", -2.0, 0.5, seed=9)
    dy = np.random.default_rng(9).standard_normal((B, T, H, D)).astype(np.float32)
    got = _run(d, "bf16", dy)
    ref = gated_delta_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dy)
    _compare(got, ref, TOL["bf16"])


def test_bwd_empty_sequence_passes_the_state_gradient_through():
    say("bwd T=0")
    B, H, D = 2, 3, 32
    dST = np.random.default_rng(4).standard_normal((B, H, D, D)).astype(np.float32)
    z = torch.zeros((B, 0, H, D), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((B, 0, H), device="cuda")
    out = gdn.gdn_prefill_bwd(z, z, z, g, g, torch.zeros((B, 0, H, D), device="cuda"), None, dev(dST))
    np.testing.assert_array_equal(host(out[5]), dST.astype(np.float64))
    out = gdn.gdn_prefill_bwd(z, z, z, g, g, torch.zeros((B, 0, H, D), device="cuda"))
    np.testing.assert_array_equal(host(out[5]), np.zeros((B, H, D, D)))


def test_bwd_4k_tokens():
    """4096 tokens (64 chunks) of the short-prefill workload's distributions, 4 heads."""
    say("bwd T=4096")
    d = config_prefill_inputs(1, T=4096, H=4, B=1)
    rng = np.random.default_rng(41)
    dy = rng.standard_normal(d["v"].shape).astype(np.float32)
    dST = rng.standard_normal((1, 4, 128, 128)).astype(np.float32)
    got = _run(d, "bf16", dy, None, dST)
    ref = gated_delta_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dy, None, dST)
    _compare(got, ref, TOL["bf16"])


@pytest.mark.timeout(900)
def test_bwd_long_workload_full_launch_all_heads():
    """The long-prefill shape (B=1, H=32, T=32768, d=128, bf16) in one launch;
    every head checked against the oracle over all 32768 tokens."""
    say("bwd long workload, all heads")
    d = config_prefill_inputs(2)
    rng = np.random.default_rng(42)
    dy = rng.standard_normal(d["v"].shape).astype(np.float32)
    got = _run(d, "bf16", dy)
    say("bwd long workload: oracle over all 32 heads")
    ref = oracle_pool.backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dy)
    _compare(got, ref, TOL["bf16"])
