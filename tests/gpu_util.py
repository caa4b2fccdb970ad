"""Helpers for the GPU parity tests: move seeded numpy inputs to the GPU and
compare GPU results with the float64 oracle."""

import sys

import numpy as np
import torch

from oracle import rel_err

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
