"""Helpers for the GPU parity tests: move seeded numpy inputs to the GPU and
compare GPU results with the float64 oracle."""

import os
import sys

import numpy as np
import torch

from oracle import rel_err
from tests import oracle_pool

# On a machine with a GPU, start the oracle pool's fork server now, while this
# process has no GPU context yet (test modules import this one at collection).
if os.path.exists("/dev/kfd") and not torch.cuda.is_initialized():
    oracle_pool.start_server()

# max |gpu - oracle| / rms(oracle) bounds, per input dtype
TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x, dtype="f32"):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def host(t):
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, got, ref, tol):
    err = rel_err(got, ref)
    say(f"    {name}: max|d|/rms = {err:.3e} (bound {tol:.0e})")
    assert np.all(np.isfinite(got)), f"{name} has non-finite values"
    assert err <= tol, f"{name}: {err:.3e} > {tol:.0e}"
    return err


def prefill(q, k, v, alpha, beta, initial_state=None, **kw):
    """gdn_prefill_fwd with a workspace of its own (or the one passed), followed
    by a check of the call's device status word (gdn_prefill_status: no
    non-finite y or state)."""
    import linear_attention_recurrence_rule_amd as gdn
    B, T, H, dk = q.shape
    need = gdn.gdn_prefill_workspace_bytes(B, T, H, dk, v.shape[-1], q.dtype)
    ws = kw.pop("workspace", None)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = gdn.gdn_prefill_fwd(q, k, v, alpha, beta, initial_state, workspace=ws, **kw)
    if ws is not None:
        gdn.gdn_prefill_status(ws, stream=kw.get("stream"))
    return out
