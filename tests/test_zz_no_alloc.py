"""gdn_prefill_fwd_noalloc (scratch in the library's static per-GPU array)
against gdn_prefill_fwd with a caller workspace, on two calls in a row, the
second smaller than the first, and both against the float64 oracle."""

import numpy as np
import pytest
import torch

from oracle import gated_delta_recurrence
from tests.gpu_util import TOL, check, dev, host, say
from workloads import prefill_inputs
import linear_attention_recurrence_rule_amd as gdn

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_the_workspace_call(dtype):
    # (B, T, H, d_k, d_v): the first call fills more of the array than the
    # second, so stale contents of the larger call sit beyond the smaller one
    cases = [(2, 1000, 8, 128, 128, 1), (1, 300, 3, 64, 128, 2)]
    for B, T, H, dk, dv, seed in cases:
        say(f"noalloc B={B} T={T} H={H} dk={dk} dv={dv} {dtype}")
        d = prefill_inputs(B, T, H, dk, dv, dtype, -1.0, 0.5, seed=seed, state_std=0.05)
        args = [dev(d[x], dtype) for x in ("q", "k", "v")] + [dev(d["alpha"]), dev(d["beta"])]
        s0 = dev(d["initial_state"])
        y_ws, S_ws = gdn.gdn_prefill_fwd(*args, s0, scale=0.75)
        y = torch.full((B, T, H, dv), float("nan"), device="cuda")
        S = torch.full((B, H, dk, dv), float("nan"), device="cuda")
        gdn.gdn_prefill_fwd_noalloc(*args, s0, S, y, scale=0.75)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ws), "y differs from the workspace call"
        assert torch.equal(S, S_ws), "final state differs from the workspace call"
        y_ref, S_ref = gated_delta_recurrence(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"],
                                              0.75)
        check("noalloc y", host(y), y_ref, TOL[dtype])
        check("noalloc state", host(S), S_ref, TOL[dtype])


def test_noalloc_in_place_state_and_oversize_rejection():
    say("noalloc in place, oversize")
    d = prefill_inputs(1, 130, 2, 128, 128, "bf16", -1.0, 0.5, seed=9, state_std=0.05)
    args = [dev(d[x], "bf16") for x in ("q", "k", "v")] + [dev(d["alpha"]), dev(d["beta"])]
    state = dev(d["initial_state"])
    y = torch.empty((1, 130, 2, 128), device="cuda")
    gdn.gdn_prefill_fwd_noalloc(*args, state, state, y)
    y_ref, S_ref = gated_delta_recurrence(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"])
    check("in-place y", host(y), y_ref, TOL["bf16"])
    check("in-place state", host(state), S_ref, TOL["bf16"])
    # one (sequence, head, chunk) unit more than the array holds: refused on the host
    T_big = 18725 * 64
    q = torch.empty((1, T_big, 1, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((1, T_big, 1), device="cuda")
    with pytest.raises(gdn.GdnError) as err:
        gdn.gdn_prefill_fwd_noalloc(q, q, q, g, g, None, None, torch.empty((1, T_big, 1, 128), device="cuda"))
    assert err.value.status == 7
