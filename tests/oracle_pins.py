"""Checks that pin a gated-delta-rule implementation to what the pages and the
mathematics fix, independently of the implementation's own formula.

Each ``pin_*`` takes ``impl(q, k, v, alpha, beta, initial_state=None,
scale=1.0) -> (y, final_state)`` with the shapes of
oracle.gated_delta_recurrence, and returns the largest deviation it saw
(float64).  The tests assert the oracle passes every pin; the mutation test
plants plausible mistakes in copies of the oracle and asserts that some pin
catches each one.

Sources: slinene ai-papers-daily page, Module A (delta form; printed "compact"
form; alpha in (0,1) controls state lifetime; repeated keys update an existing
association instead of accumulating); paper.rainbus.top digest, prerequisites
(targeted erase-write, fixed-size state) and method step (1) (compact form
alpha (I - beta k k^T) S + beta k v^T).
"""

import numpy as np
import torch

RNG_SEED = 1234


def _rand_inputs(rng, B=2, T=9, H=3, dk=5, dv=4, alpha=None, beta=None, s0=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    a = rng.uniform(0.2, 0.99, (B, T, H)) if alpha is None else np.full((B, T, H), alpha)
    b = rng.uniform(0.05, 0.95, (B, T, H)) if beta is None else np.full((B, T, H), beta)
    S0 = rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, a, b, S0


def _dense_step_p1(S, k, v, a, b):
    """rainbus digest, method step (1): alpha (I - beta k k^T) S + beta k v^T."""
    dk = k.shape[0]
    M = a * (np.eye(dk) - b * np.outer(k, k))
    return M @ S + b * np.outer(k, v)


def _dense_step_p3(S, k, v, a, b):
    """slinene page, Module A, printed compact form: (alpha I - beta k k^T) S + beta k v^T."""
    dk = k.shape[0]
    return (a * np.eye(dk) - b * np.outer(k, k)) @ S + b * np.outer(k, v)


def pin_compact_form(impl):
    """The delta form equals the digest's compact form, state and outputs
    (one rectangular and one square state shape)."""
    return max(_compact_form_case(impl, 5, 4), _compact_form_case(impl, 4, 4))


def _compact_form_case(impl, dk, dv):
    rng = np.random.default_rng(RNG_SEED + dk * 10 + dv)
    q, k, v, a, b, S0 = _rand_inputs(rng, dk=dk, dv=dv)
    y, S = impl(q, k, v, a, b, initial_state=S0)
    B, T, H, _ = q.shape
    err = 0.0
    for bb in range(B):
        for h in range(H):
            St = S0[bb, h].copy()
            for t in range(T):
                St = _dense_step_p1(St, k[bb, t, h], v[bb, t, h], a[bb, t, h], b[bb, t, h])
                err = max(err, np.max(np.abs(St.T @ q[bb, t, h] - y[bb, t, h])))
            err = max(err, np.max(np.abs(St - S[bb, h])))
    return err


def pin_p3_form_only_at_alpha_one(impl):
    """The slinene page's printed compact form agrees with the delta form when
    alpha = 1, and otherwise differs by exactly -beta (1 - alpha) k k^T S_{t-1}.

    Returns the larger of: the alpha = 1 disagreement, and the deviation of the
    one-step difference from that term.
    """
    rng = np.random.default_rng(RNG_SEED + 1)
    q, k, v, a, b, S0 = _rand_inputs(rng, B=1, H=1, T=6, alpha=1.0)
    y, S = impl(q, k, v, a, b, initial_state=S0)
    St = S0[0, 0].copy()
    for t in range(q.shape[1]):
        St = _dense_step_p3(St, k[0, t, 0], v[0, t, 0], 1.0, b[0, t, 0])
    err = np.max(np.abs(St - S[0, 0]))
    q, k, v, a, b, S0 = _rand_inputs(rng, B=1, H=1, T=1)
    _, S1 = impl(q, k, v, a, b, initial_state=S0)
    kk, aa, bb = k[0, 0, 0], a[0, 0, 0], b[0, 0, 0]
    p3 = _dense_step_p3(S0[0, 0], kk, v[0, 0, 0], aa, bb)
    expected_gap = -bb * (1.0 - aa) * np.outer(kk, kk) @ S0[0, 0]
    err = max(err, np.max(np.abs((p3 - S1[0, 0]) - expected_gap)))
    return err


def pin_pure_decay(impl):
    """beta = 0: S_T = (prod alpha) S_0 and y_t = (prod_{i<=t} alpha_i) S_0^T q_t."""
    rng = np.random.default_rng(RNG_SEED + 2)
    q, k, v, a, b, S0 = _rand_inputs(rng, beta=0.0)
    y, S = impl(q, k, v, a, b, initial_state=S0)
    cum = np.cumprod(a, axis=1)                                     # [B, T, H]
    y_ref = cum[..., None] * np.einsum("bhkv,bthk->bthv", S0, q)
    S_ref = cum[:, -1, :, None, None] * S0
    return max(np.max(np.abs(y - y_ref)), np.max(np.abs(S - S_ref)))


def pin_orthonormal_retrieval(impl):
    """alpha = beta = 1 with orthonormal keys: every written key recalls its
    value exactly, directions never written keep the initial state's
    association, and rewriting a key replaces only that key's value."""
    rng = np.random.default_rng(RNG_SEED + 3)
    dk, dv, T = 8, 3, 5
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = basis[:, :T].T                                             # T orthonormal rows
    spare = basis[:, T:].T                                            # never written
    v = rng.standard_normal((T, dv))
    S0 = rng.standard_normal((dk, dv))
    q = rng.standard_normal((T, dk))
    ones = np.ones((1, T, 1))
    _, S = impl(q[None, :, None], keys[None, :, None], v[None, :, None], ones, ones,
                initial_state=S0[None, None])
    S = S[0, 0]
    err = np.max(np.abs(keys @ S - v))
    err = max(err, np.max(np.abs(spare @ S - spare @ S0)))
    # rewrite key 2 with a new value: key 2 changes, every other key is kept
    v_new = rng.standard_normal((1, dv))
    one = np.ones((1, 1, 1))
    _, S2 = impl(q[None, :1, None], keys[None, 2:3, None], v_new[None, :, None], one, one,
                 initial_state=S[None, None])
    S2 = S2[0, 0]
    err = max(err, np.max(np.abs(keys[2] @ S2 - v_new[0])))
    others = [i for i in range(T) if i != 2]
    err = max(err, np.max(np.abs(keys[others] @ S2 - v[others])))
    return err


def pin_lms_step(impl):
    """alpha = 1: one step is one gradient-descent step of size beta on
    L(S) = 1/2 ||S^T k - v||^2 (the Widrow-Hoff delta rule); the gradient is
    taken by torch autograd in float64."""
    rng = np.random.default_rng(RNG_SEED + 4)
    q, k, v, a, b, S0 = _rand_inputs(rng, B=1, H=1, T=1, alpha=1.0)
    _, S1 = impl(q, k, v, a, b, initial_state=S0)
    St = torch.tensor(S0[0, 0], dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k[0, 0, 0], dtype=torch.float64)
    vt = torch.tensor(v[0, 0, 0], dtype=torch.float64)
    loss = 0.5 * torch.sum((St.T @ kt - vt) ** 2)
    (grad,) = torch.autograd.grad(loss, St)
    ref = S0[0, 0] - b[0, 0, 0] * grad.numpy()
    return np.max(np.abs(S1[0, 0] - ref))


def pin_scalar_closed_form(impl):
    """d_k = d_v = 1: s_t = a_t s_{t-1} + beta_t k_t v_t with
    a_t = alpha_t (1 - beta_t k_t^2); closed form
    s_t = P_t s_0 + sum_{i<=t} (P_t / P_i) beta_i k_i v_i, P_t = prod_{j<=t} a_j,
    evaluated with cumulative products and sums (|k_t| <= 0.9 keeps every
    a_t away from zero, so the divisions are safe)."""
    rng = np.random.default_rng(RNG_SEED + 5)
    T = 12
    k = rng.uniform(0.3, 0.9, T) * rng.choice([-1.0, 1.0], T)
    q = rng.standard_normal(T)
    v = rng.standard_normal(T)
    a = rng.uniform(0.3, 0.95, T)
    b = rng.uniform(0.1, 0.9, T)
    s0 = 0.7
    y, S = impl(q[None, :, None, None], k[None, :, None, None], v[None, :, None, None],
                a[None, :, None], b[None, :, None], initial_state=np.full((1, 1, 1, 1), s0))
    coef = a * (1.0 - b * k * k)
    P = np.cumprod(coef)
    drive = b * k * v
    s = P * s0 + P * np.cumsum(drive / P)
    return max(np.max(np.abs(y[0, :, 0, 0] - s * q)), abs(S[0, 0, 0, 0] - s[-1]))


def pin_brute_force_unrolled(impl):
    """Tiny shapes: S_t = (M_t ... M_1) S_0 + sum_i (M_t ... M_{i+1}) beta_i k_i v_i^T
    with dense M_j = alpha_j (I - beta_j k_j k_j^T), every product formed
    explicitly; y_t = S_t^T q_t."""
    rng = np.random.default_rng(RNG_SEED + 6)
    q, k, v, a, b, S0 = _rand_inputs(rng, B=1, H=2, T=6, dk=3, dv=2)
    y, S = impl(q, k, v, a, b, initial_state=S0)
    err = 0.0
    for h in range(2):
        M = [a[0, j, h] * (np.eye(3) - b[0, j, h] * np.outer(k[0, j, h], k[0, j, h]))
             for j in range(6)]
        for t in range(6):
            prod_all = np.eye(3)
            for j in range(t + 1):
                prod_all = M[j] @ prod_all
            St = prod_all @ S0[0, h]
            for i in range(t + 1):
                tail = np.eye(3)
                for j in range(i + 1, t + 1):
                    tail = M[j] @ tail
                St = St + tail @ (b[0, i, h] * np.outer(k[0, i, h], v[0, i, h]))
            err = max(err, np.max(np.abs(St.T @ q[0, t, h] - y[0, t, h])))
        err = max(err, np.max(np.abs(St - S[0, h])))
    return err


def pin_linearity(impl):
    """The map (S_0, V) -> (y, S_T) is linear for fixed q, k, alpha, beta."""
    rng = np.random.default_rng(RNG_SEED + 7)
    q, k, v1, a, b, S1 = _rand_inputs(rng)
    v2 = rng.standard_normal(v1.shape)
    S2 = rng.standard_normal(S1.shape)
    c1, c2 = 0.7, -1.3
    ya, Sa = impl(q, k, v1, a, b, initial_state=S1)
    yb, Sb = impl(q, k, v2, a, b, initial_state=S2)
    yc, Sc = impl(q, k, c1 * v1 + c2 * v2, a, b, initial_state=c1 * S1 + c2 * S2)
    return max(np.max(np.abs(yc - (c1 * ya + c2 * yb))), np.max(np.abs(Sc - (c1 * Sa + c2 * Sb))))


def pin_column_separability(impl):
    """Each value column evolves on its own: running on a subset of the columns
    of V and S_0 gives those columns of y and S_T."""
    rng = np.random.default_rng(RNG_SEED + 8)
    q, k, v, a, b, S0 = _rand_inputs(rng, dv=6)
    y, S = impl(q, k, v, a, b, initial_state=S0)
    cols = [1, 4, 5]
    ys, Ss = impl(q, k, v[..., cols], a, b, initial_state=S0[..., cols])
    return max(np.max(np.abs(ys - y[..., cols])), np.max(np.abs(Ss - S[..., cols])))


def pin_causality(impl):
    """Changing tokens after t0 leaves y_0 .. y_t0 unchanged."""
    rng = np.random.default_rng(RNG_SEED + 9)
    q, k, v, a, b, S0 = _rand_inputs(rng, T=10)
    y1, _ = impl(q, k, v, a, b, initial_state=S0)
    t0 = 5
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    a2, b2 = a.copy(), b.copy()
    q2[:, t0 + 1:] = np.roll(q2[:, t0 + 1:], 1, axis=-1)
    k2[:, t0 + 1:] = -k2[:, t0 + 1:]
    v2[:, t0 + 1:] += 3.0
    a2[:, t0 + 1:] = 0.5
    b2[:, t0 + 1:] = 0.9
    y2, _ = impl(q2, k2, v2, a2, b2, initial_state=S0)
    return np.max(np.abs(y1[:, :t0 + 1] - y2[:, :t0 + 1]))


def pin_segment_composition(impl):
    """Running [0, T1) then [T1, T) from the carried state equals one pass."""
    rng = np.random.default_rng(RNG_SEED + 10)
    q, k, v, a, b, S0 = _rand_inputs(rng, T=11)
    y, S = impl(q, k, v, a, b, initial_state=S0)
    T1 = 4
    y1, Sm = impl(q[:, :T1], k[:, :T1], v[:, :T1], a[:, :T1], b[:, :T1], initial_state=S0)
    y2, S2 = impl(q[:, T1:], k[:, T1:], v[:, T1:], a[:, T1:], b[:, T1:], initial_state=Sm)
    return max(np.max(np.abs(np.concatenate([y1, y2], axis=1) - y)), np.max(np.abs(S2 - S)))


def pin_hand_example(impl, fixture):
    """The four-token example worked by hand in tests/golden/hand_example.json."""
    r = fixture["recurrence"]
    k = np.array(r["k"], dtype=np.float64)[None, :, None]
    q = np.array(r["q"], dtype=np.float64)[None, :, None]
    v = np.array(r["v"], dtype=np.float64)[None, :, None]
    a = np.array(r["alpha"], dtype=np.float64)[None, :, None]
    b = np.array(r["beta"], dtype=np.float64)[None, :, None]
    y, S = impl(q, k, v, a, b)
    return max(np.max(np.abs(y[0, :, 0] - np.array(r["y"]))),
               np.max(np.abs(S[0, 0] - np.array(r["final_state"]))))


RECURRENCE_PINS = [
    pin_compact_form,
    pin_p3_form_only_at_alpha_one,
    pin_pure_decay,
    pin_orthonormal_retrieval,
    pin_lms_step,
    pin_scalar_closed_form,
    pin_brute_force_unrolled,
    pin_linearity,
    pin_column_separability,
    pin_causality,
    pin_segment_composition,
]
