"""gdn_gated_rmsnorm on the GPU against the float64 oracle epilogue."""

import numpy as np
import pytest

from oracle import gated_rmsnorm
from tests.gpu_util import check, dev, host, say
from workloads import round_to_bf16
import linear_attention_recurrence_rule_amd as gdn

pytestmark = pytest.mark.gpu

# float32 output: a d_v-term mean of squares and a sigmoid in float32 (~1e-6).
# bfloat16 output: one rounding to 8 significant bits, |d| <= 2^-9 |o|, so the
# bound scales with max|o| / rms(o) (a few units here): 2e-2.
NORM_TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.mark.parametrize("dv", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_weight", [False, True])
def test_gated_rmsnorm(dv, dtype, with_weight):
    say(f"norm dv={dv} {dtype} weight={with_weight}")
    rng = np.random.default_rng(dv)
    rows = 1000 + dv          # not a multiple of the rows per workgroup
    y = (rng.standard_normal((rows, dv)) * rng.uniform(0.1, 3, (rows, 1))).astype(np.float32)
    z = rng.standard_normal((rows, dv)).astype(np.float32)
    if dtype == "bf16":
        z = round_to_bf16(z)
    w = (0.1 * rng.standard_normal(dv)).astype(np.float32) if with_weight else None
    out = gdn.gdn_gated_rmsnorm(dev(y), dev(z, dtype), None if w is None else dev(w), eps=1e-6)
    ref = gated_rmsnorm(y, z, w, 1e-6)
    got = host(out)
    check("out", got, ref, NORM_TOL[dtype])
    if dtype == "bf16":
        # element by element: the float32 result rounded once to bfloat16 (8
        # significant bits), so within 2^-8 of the exact value, relatively,
        # plus the float32 error
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) * (1 + 1e-4) + 1e-30)


def test_gated_rmsnorm_zero_rows():
    import torch
    y = torch.zeros(0, 128, device="cuda")
    out = gdn.gdn_gated_rmsnorm(y, y.clone())
    assert out.shape == (0, 128)


def test_gated_rmsnorm_four_dim_prefill_layout():
    """The prefill output [B, T, H, d_v] as B*T*H rows."""
    say("norm 4-d")
    rng = np.random.default_rng(5)
    y = rng.standard_normal((2, 37, 3, 128)).astype(np.float32)
    z = round_to_bf16(rng.standard_normal(y.shape))
    out = gdn.gdn_gated_rmsnorm(dev(y), dev(z, "bf16"))
    check("out", host(out), gated_rmsnorm(y, z, None, 1e-6), NORM_TOL["bf16"])
