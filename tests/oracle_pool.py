"""Run the float64 oracle on independent (sequence, head) slices in parallel.

Heads and sequences are independent under the recurrence, so the oracle can
be evaluated one (b, h) slice at a time in worker processes and the slices
reassembled; the arithmetic is exactly the oracle's.  This module imports no
GPU code: the workers are forked by a fork server that the GPU tests start
before anything touches the GPU (start_server), so no process with a GPU
context is ever forked.  Without a started server every call runs in-process,
one slice after another.
"""

import atexit
import concurrent.futures
import multiprocessing
import os

import numpy as np

from oracle import gated_delta_backward, gated_delta_decode_step, gated_delta_recurrence

_CTX = None
_POOL = None
MAX_WORKERS = 16


def start_server():
    """Start the fork server that will fork the workers.  Call it before the
    process initialises the GPU; later calls are no-ops."""
    global _CTX
    if _CTX is not None:
        return
    ctx = multiprocessing.get_context("forkserver")
    ctx.set_forkserver_preload(["numpy", "oracle"])
    from multiprocessing import forkserver
    forkserver.ensure_running()
    _CTX = ctx


def _pool():
    global _POOL
    if _CTX is None:
        return None
    if _POOL is None:
        n = max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0))))
        _POOL = concurrent.futures.ProcessPoolExecutor(max_workers=n, mp_context=_CTX)
        atexit.register(_shutdown)
    return _POOL


def _shutdown():
    global _POOL
    if _POOL is not None:
        _POOL.shutdown(wait=True)
        _POOL = None


def _map(fn, tasks):
    pool = _pool()
    if pool is None:
        return [fn(*t) for t in tasks]
    return [f.result() for f in [pool.submit(fn, *t) for t in tasks]]


def map_tasks(fn, tasks):
    """fn(*t) for each tuple t of `tasks`, in the pool when there is one (fn
    must be a module-level function of a module the workers can import)."""
    return _map(fn, tasks)


def _sl(x, b, h):
    return None if x is None else x[b:b + 1, :, h:h + 1]


def _fwd(q, k, v, alpha, beta, s0, scale):
    return gated_delta_recurrence(q, k, v, alpha, beta, s0, scale)


def recurrence(q, k, v, alpha, beta, initial_state=None, scale=1.0):
    """gated_delta_recurrence over [B, T, H, ...] inputs, one task per (b, h)."""
    B, T, H, _ = q.shape
    dv = v.shape[-1]
    pairs = [(b, h) for b in range(B) for h in range(H)]
    tasks = [(_sl(q, b, h), _sl(k, b, h), _sl(v, b, h), _sl(alpha, b, h), _sl(beta, b, h),
              None if initial_state is None else initial_state[b:b + 1, h:h + 1], scale) for b, h in pairs]
    res = _map(_fwd, tasks)
    y = np.empty((B, T, H, dv))
    S = np.empty((B, H, q.shape[-1], dv))
    for (b, h), (yb, Sb) in zip(pairs, res):
        y[b, :, h] = yb[0, :, 0]
        S[b, h] = Sb[0, 0]
    return y, S


def _bwd(q, k, v, alpha, beta, dy, s0, dST):
    return gated_delta_backward(q, k, v, alpha, beta, dy, s0, dST)


def backward(q, k, v, alpha, beta, dy, initial_state=None, d_final_state=None):
    """gated_delta_backward over [B, T, H, ...] inputs, one task per (b, h);
    returns the oracle's tuple (dq, dk, dv, dalpha, dbeta, d_initial_state)."""
    B, T, H, _ = q.shape
    pairs = [(b, h) for b in range(B) for h in range(H)]
    tasks = [(_sl(q, b, h), _sl(k, b, h), _sl(v, b, h), _sl(alpha, b, h), _sl(beta, b, h), _sl(dy, b, h),
              None if initial_state is None else initial_state[b:b + 1, h:h + 1],
              None if d_final_state is None else d_final_state[b:b + 1, h:h + 1]) for b, h in pairs]
    res = _map(_bwd, tasks)
    outs = [np.empty(q.shape), np.empty(k.shape), np.empty(v.shape), np.empty(alpha.shape),
            np.empty(beta.shape), np.empty((B, H, q.shape[-1], v.shape[-1]))]
    for (b, h), r in zip(pairs, res):
        for i in range(5):
            outs[i][b, :, h] = r[i][0, :, 0]
        outs[5][b, h] = r[5][0, 0]
    return tuple(outs)


def _dec(q, k, v, alpha, beta, S, scale):
    return gated_delta_decode_step(q, k, v, alpha, beta, S, scale)


def decode_step(q, k, v, alpha, beta, state, scale=1.0, parts=None):
    """gated_delta_decode_step over [N, H, ...] inputs, split over N into at
    most `parts` tasks (default: one per worker)."""
    N = q.shape[0]
    parts = parts or MAX_WORKERS
    cuts = np.linspace(0, N, min(parts, N) + 1).astype(int)
    tasks = [(q[a:b], k[a:b], v[a:b], alpha[a:b], beta[a:b], state[a:b], scale)
             for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    res = _map(_dec, tasks)
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])
