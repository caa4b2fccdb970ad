"""gdn_frontend_fwd on the GPU against the float64 front-end oracle, and the
front end feeding the prefill against the oracle chain."""

import numpy as np
import pytest
import torch

from oracle import gated_delta_recurrence, gdn_frontend
from tests.gpu_util import TOL, check, dev, host, say
from workloads import frontend_inputs, round_to_bf16
import linear_attention_recurrence_rule_amd as gdn

pytestmark = pytest.mark.gpu

# elementwise bounds: bf16 outputs are one bf16 rounding (2^-8 relative) off the
# exact values, float32 ones a few float32 roundings and the fast exponential
BOUND = {"bf16": (2.0 ** -8, 1e-6), "f32": (2e-5, 1e-6)}
GATE_RTOL = 2e-5


def _to_dev(d, dtype):
    keys = ("q_proj", "k_proj", "v_proj", "q_hist", "k_hist", "v_hist")
    return {key: dev(val, dtype if key in keys else "f32") for key, val in d.items()}


def _run(d, dtype, eps=1e-6):
    g = _to_dev(d, dtype)
    return gdn.gdn_frontend_fwd(g["q_proj"], g["k_proj"], g["v_proj"], g["conv_q"], g["conv_k"], g["conv_v"],
                                g["a_logit"], g["b_logit"], g["A"], g["b_alpha"], g.get("q_hist"),
                                g.get("k_hist"), g.get("v_hist"), eps=eps)


def _ref(d, eps=1e-6):
    return gdn_frontend(d["q_proj"], d["k_proj"], d["v_proj"], d["conv_q"], d["conv_k"], d["conv_v"],
                        d["a_logit"], d["b_logit"], d["A"], d["b_alpha"], d.get("q_hist"), d.get("k_hist"),
                        d.get("v_hist"), eps=eps)


def _compare(got, ref, dtype, label=""):
    rtol, atol = BOUND[dtype]
    names = ("q", "k", "v", "alpha", "beta")
    for name, g, r in zip(names, got, ref):
        gh = host(g)
        assert np.all(np.isfinite(gh)), f"{label}{name} has non-finite values"
        if name in ("alpha", "beta"):
            err = np.max(np.abs(gh - r) / np.maximum(np.abs(r), 1e-30)) if r.size else 0.0
            say(f"    {label}{name}: max rel {err:.2e}")
            assert err <= GATE_RTOL
        else:
            excess = np.abs(gh - r) - (rtol * np.abs(r) + atol)
            say(f"    {label}{name}: max |d| {np.max(np.abs(gh - r)) if r.size else 0:.2e}")
            assert np.all(excess <= 0), f"{label}{name}: bound exceeded by {np.max(excess):.2e}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 32), (16, 128), (32, 16)])
@pytest.mark.parametrize("width", [1, 2, 4])
def test_frontend_matches_oracle(dtype, dk, dv, width):
    say(f"frontend dtype={dtype} dk={dk} dv={dv} W={width}")
    d = frontend_inputs(2, 77, 5, dk, dv, dtype, A=-1.0, width=width, seed=dk + dv + width)
    _compare(_run(d, dtype), _ref(d), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_frontend_history_and_segments(dtype):
    """Rows before t = 0 from the caller, and two segments chained through them."""
    say(f"frontend history dtype={dtype}")
    d = frontend_inputs(2, 70, 3, 64, 64, dtype, A=-2.0, width=4, seed=11, history=True)
    _compare(_run(d, dtype), _ref(d), dtype, "with history: ")
    # split at t = 29: the second segment's history is the first segment's last 3 rows
    t1 = 29
    first = {key: (val[:, :t1] if val.ndim >= 3 and val.shape[1] == 70 else val) for key, val in d.items()}
    second = {key: (val[:, t1:] if val.ndim >= 3 and val.shape[1] == 70 else val) for key, val in d.items()}
    for s in ("q", "k", "v"):
        second[f"{s}_hist"] = d[f"{s}_proj"][:, t1 - 3:t1]
    ref = _ref(d)
    a, b = _run(first, dtype), _run(second, dtype)
    joined = [torch.cat([x, y], dim=1) for x, y in zip(a, b)]
    _compare(joined, ref, dtype, "segmented: ")


def test_frontend_zero_length():
    d = frontend_inputs(1, 0, 2, 32, 32, "bf16")
    out = _run(d, "bf16")
    assert all(t.numel() == 0 for t in out)


def test_frontend_then_prefill_matches_oracle_chain():
    """Front end on the GPU feeding the GPU prefill, against the oracle front
    end feeding the oracle recurrence (bf16 recurrence inputs in both)."""
    say("frontend -> prefill")
    d = frontend_inputs(1, 300, 4, 128, 128, "bf16", A=-2.0, width=4, seed=21)
    q, k, v, alpha, beta = _run(d, "bf16")
    y, S = gdn.gdn_prefill_fwd(q, k, v, alpha, beta)
    rq, rk, rv, ra, rb = _ref(d)
    # the recurrence oracle takes the bf16 values the GPU front end produced
    # (they agree with the oracle's to one rounding, checked above); the gates
    # in float32 as the API carries them
    y_ref, S_ref = gated_delta_recurrence(host(q), host(k), host(v), host(alpha), host(beta))
    check("y", host(y), y_ref, TOL["bf16"])
    check("state", host(S), S_ref, TOL["bf16"])
    # and the chain is close to the exact one (inputs rounded to bf16 once)
    y_exact, _ = gated_delta_recurrence(round_to_bf16(rq), round_to_bf16(rk), round_to_bf16(rv),
                                        ra.astype(np.float32), rb.astype(np.float32))
    check("y vs exact chain", host(y), y_exact, TOL["bf16"])


def test_frontend_long_shape_sampled():
    """The long-prefill shape (B=1, T=32768, H=32, d=128) in one launch, compared
    with the oracle on sampled heads and token windows."""
    say("frontend long shape")
    B, T, H, dd = 1, 32768, 32, 128
    d = frontend_inputs(B, T, H, dd, dd, "bf16", A=-2.0, width=4, seed=2)
    got = [host(t) for t in _run(d, "bf16")]
    for h in (0, 17, 31):
        for t0 in (0, 12345, T - 40):
            sl = slice(max(t0 - 3, 0), t0 + 40)
            sub = {key: (val[:, sl][:, :, [h]] if val.ndim >= 3 and val.shape[1] == T else val) for key, val in d.items()}
            for key in ("conv_q", "conv_k", "conv_v", "A", "b_alpha"):
                sub[key] = d[key][[h]]
            ref = _ref(sub)
            lo = t0 - sl.start
            rtol, atol = BOUND["bf16"]
            for i, name in enumerate(("q", "k", "v")):
                g = got[i][:, sl][:, lo:, [h]]
                r = ref[i][:, lo:]
                assert np.all(np.abs(g - r) <= rtol * np.abs(r) + atol), f"{name} h={h} t0={t0}"
            for i, name in ((3, "alpha"), (4, "beta")):
                g = got[i][:, sl][:, lo:, [h]]
                r = ref[i][:, lo:]
                assert np.max(np.abs(g - r) / np.abs(r)) <= GATE_RTOL, f"{name} h={h} t0={t0}"
