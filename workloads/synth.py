"""Seeded generators for the five GDN workloads.

The workloads stand in for the long-context training sequences the pages
describe (4K pre-training, 32K extension, 256K continued pre-training; slinene
page, overall data flow and Module B) with seeded Gaussian tensors.  The pages
give no head count or head size; the shapes below are the ones this library is
measured on.

Recipe, per token and head:
  q, k ~ N(0, 1), then divided by their own L2 norm in float64 (the mixer
        L2-normalises q and k before the recurrence: slinene page, Module A;
        rainbus digest, method step (1));
  v, z ~ N(0, 1);
  beta  = sigmoid(N(0, 1));
  alpha = exp(-exp(A) * softplus(N(0, 1) + b)), the decay parameterisation
        of slinene page Module A, with the config's A and b = 0.5;
  q, k, v, z are rounded to bfloat16 (round to nearest even) unless the
  config is float32; alpha, beta and states stay float32.
Arrays are returned as float32 numpy arrays whose values are exactly the
values handed to the GPU (bf16 values are exactly representable in float32).

Seeds: a sequence of at most SEGMENT tokens draws from
numpy.random.default_rng(seed); longer ones draw segment s (SEGMENT tokens
each) from default_rng([seed, s]).  An optional prefill initial state draws
from default_rng([seed, STATE_STREAM]).  Draw order inside a segment: q, k, v,
beta-logit, alpha-logit, z.  Decode step j draws from default_rng([seed, j]);
the decode initial state draws from default_rng(seed); a block of draft
tokens for multi-token decode draws from default_rng([seed, MTP_STREAM, block]).
"""

import numpy as np

SEGMENT = 4096
STATE_STREAM = 2**31 - 1     # second seed word of the initial-state stream

CONFIGS = {
    0: dict(name="tiny_oracle_check", kind="prefill", B=1, H=1, T=64, dk=16, dv=16,
            dtype="f32", A=-1.0, b=0.5, seed=0, z=False),
    1: dict(name="prefill_short", kind="prefill", B=4, H=16, T=4096, dk=128, dv=128,
            dtype="bf16", A=-1.0, b=0.5, seed=1, z=True),
    2: dict(name="prefill_long", kind="prefill", B=1, H=32, T=32768, dk=128, dv=128,
            dtype="bf16", A=-2.0, b=0.5, seed=2, z=True),
    3: dict(name="decode", kind="decode", N=256, H=32, steps=1000, dk=128, dv=128,
            dtype="bf16", A=-1.0, b=0.5, seed=3, state_std=0.02),
    4: dict(name="very_long_segmented", kind="prefill", B=1, H=16, T=262144, dk=128,
            dv=128, dtype="bf16", A=-2.0, b=0.5, seed=4, z=True, segment=SEGMENT),
}


def round_to_bf16(x):
    """Round to the nearest bfloat16 (ties to even), returned as float32."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def _cast(x, dtype):
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _unit_rows(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _softplus(u):
    return np.logaddexp(0.0, u)


def _sigmoid(u):
    return 1.0 / (1.0 + np.exp(-u))


def _draw_segment(rng, B, T, H, dk, dv, A, b, dtype, with_z):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    beta_logit = rng.standard_normal((B, T, H))
    alpha_logit = rng.standard_normal((B, T, H))
    out = dict(
        q=_cast(_unit_rows(q), dtype),
        k=_cast(_unit_rows(k), dtype),
        v=_cast(v, dtype),
        beta=_sigmoid(beta_logit).astype(np.float32),
        alpha=np.exp(-np.exp(A) * _softplus(alpha_logit + b)).astype(np.float32),
    )
    if with_z:
        out["z"] = _cast(rng.standard_normal((B, T, H, dv)), dtype)
    return out


def prefill_inputs(B, T, H, dk, dv, dtype="bf16", A=-1.0, b=0.5, seed=0, with_z=False,
                   state_std=0.0, t_begin=0):
    """Draw q, k, v, alpha, beta (and z, initial_state) for a prefill call.

    ``t_begin`` (a multiple of SEGMENT) lets callers draw tokens
    [t_begin, t_begin + T) of a long sequence without drawing the rest.
    ``state_std`` > 0 adds an N(0, state_std^2) float32 initial state drawn
    from default_rng([seed, STATE_STREAM]).
    """
    if T + t_begin <= SEGMENT and t_begin == 0:
        out = _draw_segment(np.random.default_rng(seed), B, T, H, dk, dv, A, b, dtype, with_z)
    else:
        if t_begin % SEGMENT:
            raise ValueError("t_begin must be a multiple of SEGMENT")
        parts = []
        t = t_begin
        while t < t_begin + T:
            n = min(SEGMENT, t_begin + T - t)
            rng = np.random.default_rng([seed, t // SEGMENT])
            seg = _draw_segment(rng, B, SEGMENT, H, dk, dv, A, b, dtype, with_z)
            parts.append({key: val[:, :n] for key, val in seg.items()})
            t += n
        out = {key: np.concatenate([p[key] for p in parts], axis=1) for key in parts[0]}
    if state_std > 0:
        rng = np.random.default_rng([seed, STATE_STREAM])
        out["initial_state"] = (state_std * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    return out


def config_prefill_inputs(index, T=None, H=None, B=None, t_begin=0):
    """Inputs for prefill config ``index``, optionally at a smaller T, H or B.

    A smaller shape is a smaller workload with the config's distributions,
    not a slice of the full-size draw; callers that need the full-size values
    draw the full shape (segment by segment via ``t_begin``).
    """
    c = CONFIGS[index]
    if c["kind"] != "prefill":
        raise ValueError("not a prefill config")
    return prefill_inputs(B or c["B"], T or c["T"], H or c["H"], c["dk"], c["dv"], c["dtype"],
                          c["A"], c["b"], c["seed"], c["z"], 0.0, t_begin)


def decode_initial_state(index=3, N=None, H=None):
    """Float32 N(0, state_std^2) initial states [N, H, d_k, d_v] for the decode config."""
    c = CONFIGS[index]
    N, H = N or c["N"], H or c["H"]
    rng = np.random.default_rng(c["seed"])
    return (c["state_std"] * rng.standard_normal((N, H, c["dk"], c["dv"]))).astype(np.float32)


def decode_step_inputs(step, index=3, N=None, H=None):
    """q, k, v [N, H, d], alpha, beta [N, H] for decode step ``step``."""
    c = CONFIGS[index]
    N, H = N or c["N"], H or c["H"]
    seg = _draw_segment(np.random.default_rng([c["seed"], step]), N, 1, H, c["dk"], c["dv"],
                        c["A"], c["b"], c["dtype"], False)
    return {key: val[:, 0] for key, val in seg.items()}


def frontend_inputs(B, T, H, dk, dv, dtype="bf16", A=-1.0, b=0.5, width=4, seed=0, history=False):
    """Inputs of the front end (projected streams, filters, gate logits).

    q_proj, k_proj, v_proj ~ N(0, 1) (rounded to bf16 unless dtype is f32);
    filters conv_* ~ N(0, 1/width); a_logit, b_logit ~ N(0, 1); A[h] = A and
    b_alpha[h] = b for every head, so the gates follow the workload recipe
    above; with ``history`` the width-1 rows before t = 0 are drawn too.
    Draw order: q_proj, k_proj, v_proj, conv_q, conv_k, conv_v, b_logit,
    a_logit, then the histories.
    """
    rng = np.random.default_rng([seed, 7])
    out = dict(
        q_proj=_cast(rng.standard_normal((B, T, H, dk)), dtype),
        k_proj=_cast(rng.standard_normal((B, T, H, dk)), dtype),
        v_proj=_cast(rng.standard_normal((B, T, H, dv)), dtype),
        conv_q=(rng.standard_normal((H, dk, width)) / np.sqrt(width)).astype(np.float32),
        conv_k=(rng.standard_normal((H, dk, width)) / np.sqrt(width)).astype(np.float32),
        conv_v=(rng.standard_normal((H, dv, width)) / np.sqrt(width)).astype(np.float32),
        b_logit=rng.standard_normal((B, T, H)).astype(np.float32),
        a_logit=rng.standard_normal((B, T, H)).astype(np.float32),
        A=np.full(H, A, dtype=np.float32),
        b_alpha=np.full(H, b, dtype=np.float32),
    )
    if history:
        out["q_hist"] = _cast(rng.standard_normal((B, width - 1, H, dk)), dtype)
        out["k_hist"] = _cast(rng.standard_normal((B, width - 1, H, dk)), dtype)
        out["v_hist"] = _cast(rng.standard_normal((B, width - 1, H, dv)), dtype)
    return out


MTP_STREAM = 2**31 - 2       # second seed word of the draft-block stream


def mtp_draft_inputs(rnd, K=4, index=3, N=None, H=None):
    """q, k, v [N, K, H, d], alpha, beta [N, K, H] for draft block ``rnd`` of
    the decode config: K draft tokens per sequence with the config's
    distributions, drawn from default_rng([seed, MTP_STREAM, rnd])."""
    c = CONFIGS[index]
    N, H = N or c["N"], H or c["H"]
    return _draw_segment(np.random.default_rng([c["seed"], MTP_STREAM, rnd]), N, K, H, c["dk"], c["dv"],
                         c["A"], c["b"], c["dtype"], False)


QSA_STREAM = 2**31 - 3       # second seed word of the indexer streams


def qsa_inputs(B, n, H=4, D=128, dtype="bf16", seed=0):
    """Projected indexer streams: q_proj [B, n, H, D] and k_proj [B, n, D],
    N(0, 1) (rounded to bf16 unless dtype is f32), from
    default_rng([seed, QSA_STREAM, 0])."""
    rng = np.random.default_rng([seed, QSA_STREAM, 0])
    return dict(q_proj=_cast(rng.standard_normal((B, n, H, D)), dtype),
                k_proj=_cast(rng.standard_normal((B, n, D)), dtype))


def qsa_select_inputs(B, n, r=4, H=4, D=128, dtype="bf16", seed=0):
    """Prepared indexer operands for the scoring / selection step: q [B, n, H, D]
    and pooled keys kbar [B, n // r, D].  After RMSNorm and the rotation their
    entries have unit mean square, so N(0, 1) draws (rounded to bf16 unless
    dtype is f32) stand in for them; from default_rng([seed, QSA_STREAM, 1])."""
    rng = np.random.default_rng([seed, QSA_STREAM, 1])
    return dict(q=_cast(rng.standard_normal((B, n, H, D)), dtype),
                kbar=_cast(rng.standard_normal((B, n // r, D)), dtype))
