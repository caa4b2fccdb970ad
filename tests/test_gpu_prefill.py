"""gdn_prefill_fwd on the GPU against the float64 token-by-token oracle."""

import numpy as np
import pytest
import torch

from oracle import gated_delta_recurrence
from tests.gpu_util import TOL, check, dev, host, say
from workloads import CONFIGS, SEGMENT, config_prefill_inputs, prefill_inputs
import linear_attention_recurrence_rule_amd as gdn

pytestmark = pytest.mark.gpu


def run_case(d, dtype, scale=1.0, with_state=True, tol=None):
    tol = TOL[dtype] if tol is None else tol
    s0 = d.get("initial_state") if with_state else None
    y, S = gdn.gdn_prefill_fwd(dev(d["q"], dtype), dev(d["k"], dtype), dev(d["v"], dtype),
                               dev(d["alpha"]), dev(d["beta"]),
                               None if s0 is None else dev(s0), scale=scale)
    y_ref, S_ref = gated_delta_recurrence(d["q"], d["k"], d["v"], d["alpha"], d["beta"], s0, scale)
    if y_ref.size:
        check("y", host(y), y_ref, tol)
    check("final state", host(S), S_ref, tol)


def test_config0_tiny_fp32():
    say("prefill config 0")
    run_case(config_prefill_inputs(0), "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (32, 32), (16, 16), (128, 64), (64, 128),
                                   (16, 128), (128, 32)])
def test_multi_chunk_ragged(dtype, dk, dv):
    """Several chunks plus a ragged tail, a non-zero initial state and a scale."""
    say(f"prefill dk={dk} dv={dv} {dtype}")
    d = prefill_inputs(2, 64 * 3 + 37, 3, dk, dv, dtype, -1.0, 0.5, seed=dk + dv, state_std=0.05)
    run_case(d, dtype, scale=0.5)


@pytest.mark.parametrize("T", [1, 15, 16, 31, 63, 64, 65, 128, 129])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lengths_around_chunk_edges(T, dtype):
    say(f"prefill T={T} {dtype}")
    d = prefill_inputs(1, T, 2, 128, 128, dtype, -1.0, 0.5, seed=T, state_std=0.05)
    run_case(d, dtype)


def test_zero_length_copies_state():
    say("prefill T=0")
    d = prefill_inputs(2, 0, 3, 64, 64, "bf16", -1.0, 0.5, seed=1, state_std=0.3)
    run_case(d, "bf16", tol=0.0)
    y, S = gdn.gdn_prefill_fwd(*(torch.zeros(2, 0, 3, 64, device="cuda", dtype=torch.bfloat16)
                                 for _ in range(3)),
                               torch.zeros(2, 0, 3, device="cuda"), torch.zeros(2, 0, 3, device="cuda"))
    assert float(host(S).max()) == 0.0 and float(host(S).min()) == 0.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_alpha_zero_and_one(dtype):
    """alpha = 0 wipes the state mid-chunk; alpha = 1, beta = 1 runs undecayed."""
    say(f"prefill alpha edge {dtype}")
    d = prefill_inputs(1, 200, 2, 64, 64, dtype, -1.0, 0.5, seed=11, state_std=0.2)
    d["alpha"][0, [0, 5, 63, 64, 100, 101, 199], :] = 0.0
    d["alpha"][0, 130:160, :] = 1.0
    d["beta"][0, 130:160, :] = 1.0
    run_case(d, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_beta_zero_pure_decay(dtype):
    say(f"prefill beta=0 {dtype}")
    d = prefill_inputs(1, 150, 2, 128, 128, dtype, -2.0, 0.5, seed=12, state_std=0.5)
    d["beta"][:] = 0.0
    run_case(d, dtype)


def test_final_state_in_place():
    say("prefill in place")
    d = prefill_inputs(2, 300, 4, 128, 128, "bf16", -1.0, 0.5, seed=13, state_std=0.05)
    state = dev(d["initial_state"])
    y, S = gdn.gdn_prefill_fwd(dev(d["q"], "bf16"), dev(d["k"], "bf16"), dev(d["v"], "bf16"),
                               dev(d["alpha"]), dev(d["beta"]), state, final_state=state)
    assert S.data_ptr() == state.data_ptr()
    y_ref, S_ref = gated_delta_recurrence(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["initial_state"])
    check("y", host(y), y_ref, TOL["bf16"])
    check("state", host(state), S_ref, TOL["bf16"])


def test_segments_equal_one_call():
    """Carrying the state across calls (segments not multiples of the chunk)."""
    say("prefill segments")
    d = prefill_inputs(1, 700, 4, 128, 128, "bf16", -2.0, 0.5, seed=14)
    y1, S1 = gdn.gdn_prefill_fwd(dev(d["q"], "bf16"), dev(d["k"], "bf16"), dev(d["v"], "bf16"),
                                 dev(d["alpha"]), dev(d["beta"]))
    state = None
    ys = []
    for a, b in [(0, 100), (100, 357), (357, 700)]:
        ya, state = gdn.gdn_prefill_fwd(*(dev(d[x][:, a:b], "bf16") for x in ("q", "k", "v")),
                                        dev(d["alpha"][:, a:b]), dev(d["beta"][:, a:b]), state)
        ys.append(host(ya))
    y_ref, S_ref = gated_delta_recurrence(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    check("segmented y", np.concatenate(ys, axis=1), y_ref, TOL["bf16"])
    check("segmented state", host(state), S_ref, TOL["bf16"])
    check("one-call y", host(y1), y_ref, TOL["bf16"])


def test_prefill_then_decode():
    """Decode steps continuing from a prefill state equal a longer prefill."""
    say("prefill then decode")
    d = prefill_inputs(2, 133, 3, 128, 128, "bf16", -1.0, 0.5, seed=15)
    T0 = 130
    _, state = gdn.gdn_prefill_fwd(*(dev(d[x][:, :T0], "bf16") for x in ("q", "k", "v")),
                                   dev(d["alpha"][:, :T0]), dev(d["beta"][:, :T0]))
    y_ref, S_ref = gated_delta_recurrence(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    for t in range(T0, 133):
        y = gdn.gdn_decode_step(*(dev(d[x][:, t], "bf16") for x in ("q", "k", "v")),
                                dev(d["alpha"][:, t]), dev(d["beta"][:, t]), state)
        check(f"t={t}", host(y), y_ref[:, t], TOL["bf16"])
    check("state", host(state), S_ref, TOL["bf16"])


def _sampled_heads(idx, pairs):
    c = CONFIGS[idx]
    say(f"prefill config {idx} full shape: generating")
    d = config_prefill_inputs(idx)
    say(f"prefill config {idx}: GPU run (B={c['B']} T={c['T']} H={c['H']})")
    y, S = gdn.gdn_prefill_fwd(dev(d["q"], "bf16"), dev(d["k"], "bf16"), dev(d["v"], "bf16"),
                               dev(d["alpha"]), dev(d["beta"]))
    yh, Sh = host(y), host(S)
    for b, h in pairs:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        y_ref, S_ref = gated_delta_recurrence(d["q"][sl], d["k"][sl], d["v"][sl], d["alpha"][sl],
                                              d["beta"][sl])
        check(f"(b={b}, h={h}) y", yh[sl], y_ref, TOL["bf16"])
        check(f"(b={b}, h={h}) state", Sh[b:b + 1, h:h + 1], S_ref, TOL["bf16"])


def test_config1_full_shape_sampled_heads():
    _sampled_heads(1, [(0, 0), (1, 7), (3, 15), (2, 9)])


def test_config2_full_shape_sampled_heads():
    _sampled_heads(2, [(0, 0), (0, 13), (0, 31)])


def test_config4_segmented_262k_sampled_heads():
    """The 262,144-token sequence as 64 calls of 4096 tokens, the state carried
    through the initial/final-state arguments; sampled heads are compared with
    the oracle over every token and at the end."""
    c = CONFIGS[4]
    T, H, seg = c["T"], c["H"], c["segment"]
    heads = [0, 11]
    state = None
    ref_state = None
    max_dy, sum_sq, count = 0.0, 0.0, 0
    for s in range(T // seg):
        if s % 8 == 0:
            say(f"config 4: segment {s} of {T // seg}")
        d = config_prefill_inputs(4, T=seg, t_begin=s * seg)
        y, state = gdn.gdn_prefill_fwd(dev(d["q"], "bf16"), dev(d["k"], "bf16"), dev(d["v"], "bf16"),
                                       dev(d["alpha"]), dev(d["beta"]), state)
        yh = host(y)[:, :, heads]
        hs = (slice(None), slice(None), heads)
        y_ref, ref_state = gated_delta_recurrence(d["q"][hs], d["k"][hs], d["v"][hs], d["alpha"][hs],
                                                  d["beta"][hs], ref_state)
        max_dy = max(max_dy, float(np.max(np.abs(yh - y_ref))))
        sum_sq += float(np.sum(y_ref * y_ref))
        count += y_ref.size
        assert np.all(np.isfinite(yh))
    err = max_dy / np.sqrt(sum_sq / count)
    say(f"    config 4 y over {T} tokens, heads {heads}: max|d|/rms = {err:.3e}")
    assert err <= TOL["bf16"]
    check("config 4 final state", host(state)[:, heads], ref_state, TOL["bf16"])
