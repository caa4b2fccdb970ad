"""Python binding of libgdn, the gfx950 Gated DeltaNet token-mixer library.

The functions below carry the names of the C entry points declared in
include/gdn.h and only marshal arguments: they check dtypes, shapes and
contiguity of torch tensors, allocate missing outputs with torch (device
memory is PyTorch's job here), and pass raw device pointers plus the current
HIP stream to the library.  Every step of the computation runs in the HIP
kernels.  There is no fallback: if libgdn.so is missing, loading fails with an
ImportError that says how to build it.
"""

import contextlib
import ctypes
import functools
import os

import torch

__all__ = [
    "GDN_F32", "GDN_BF16", "GdnError", "load_library", "library_path",
    "gdn_prefill_fwd", "gdn_prefill_fwd_noalloc", "gdn_prefill_workspace_bytes", "gdn_prefill_status",
    "gdn_decode_step",
    "gdn_gated_rmsnorm",
    "gdn_frontend_fwd", "gdn_decode_mtp_verify", "gdn_decode_mtp_commit", "gdn_decode_mtp_commit_verify",
    "gdn_prefill_bwd", "gdn_prefill_bwd_workspace_bytes", "gdn_qsa_prep", "gdn_qsa_select",
    "gdn_qsa_select_workspace_bytes", "gdn_status_string",
]

GDN_F32 = 0
GDN_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgdn.so"
_lib = None


def library_path():
    return os.path.join(_HERE, _LIB_NAME)


class GdnError(RuntimeError):
    """A non-zero gdn_status returned by the library."""

    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {gdn_status_string(status)} (status {status})")


def load_library():
    """Load libgdn.so from this package directory (once) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with "
                          "`python -m linear_attention_recurrence_rule_amd.build`")
    lib = ctypes.CDLL(path)
    vp, fp, i, f, lg = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_long
    sz = ctypes.c_size_t
    lib.gdn_prefill_fwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, i, i, i, i, i, i, f, vp, sz, vp]
    lib.gdn_prefill_fwd.restype = ctypes.c_int
    lib.gdn_prefill_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.gdn_prefill_workspace_bytes.restype = sz
    lib.gdn_prefill_fwd_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, i, i, i, i, i, i, f, vp]
    lib.gdn_prefill_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_prefill_status.argtypes = [vp, vp]
    lib.gdn_prefill_status.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, fp, i, i, i, i, i, f, vp]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_gated_rmsnorm.argtypes = [fp, vp, fp, f, vp, lg, i, i, vp]
    lib.gdn_gated_rmsnorm.restype = ctypes.c_int
    lib.gdn_frontend_fwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, vp, vp, vp, vp, vp, vp, fp, fp,
                                     i, i, i, i, i, i, i, f, vp]
    lib.gdn_frontend_fwd.restype = ctypes.c_int
    lib.gdn_decode_mtp_verify.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, fp, i, i, i, i, i, i, f, vp]
    lib.gdn_decode_mtp_verify.restype = ctypes.c_int
    lib.gdn_decode_mtp_commit.argtypes = [vp, fp, fp, fp, vp, fp, i, i, i, i, i, i, vp]
    lib.gdn_decode_mtp_commit.restype = ctypes.c_int
    lib.gdn_decode_mtp_commit_verify.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, fp, fp, vp,
                                                 i, i, i, i, i, i, i, f, vp]
    lib.gdn_decode_mtp_commit_verify.restype = ctypes.c_int
    lib.gdn_prefill_bwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                    i, i, i, i, i, i, f, vp, sz, vp]
    lib.gdn_prefill_bwd.restype = ctypes.c_int
    lib.gdn_prefill_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.gdn_prefill_bwd_workspace_bytes.restype = sz
    lib.gdn_qsa_prep.argtypes = [vp, vp, fp, fp, vp, vp, i, i, i, i, i, i, f, f, i, vp]
    lib.gdn_qsa_prep.restype = ctypes.c_int
    lib.gdn_qsa_select.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]
    lib.gdn_qsa_select.restype = ctypes.c_int
    lib.gdn_qsa_select_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.gdn_qsa_select_workspace_bytes.restype = sz
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def gdn_status_string(status):
    return load_library().gdn_status_string(int(status)).decode()


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _require_gpu(t, name):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")


def _stream(stream, device):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run a binding with ``stream`` (when one is given) as torch's current
    stream, so that every tensor it allocates (outputs and scratch) belongs to
    the stream its kernels run on.  The caching allocator then cannot hand a
    dropped scratch block to other work before those kernels are done with it."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        ctx = contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)
        with ctx:
            return fn(*args, stream=stream, **kwargs)
    return wrapper


def gdn_prefill_workspace_bytes(B, T, H, d_k, d_v, dtype):
    """Scratch bytes gdn_prefill_fwd needs (dtype: torch.bfloat16 or torch.float32)."""
    code = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(load_library().gdn_prefill_workspace_bytes(B, T, H, d_k, d_v, code))


def gdn_prefill_status(workspace, stream=None):
    """Synchronise ``stream`` and raise GdnError(GDN_ERR_DEVICE) if the last
    bf16 gdn_prefill_fwd call on ``workspace`` wrote a non-finite y or final
    state value (with finite inputs: an input or intermediate outside the fp16
    operand range).  Returns None when the call was clean."""
    _require_gpu(workspace, "workspace")
    st = load_library().gdn_prefill_status(_ptr(workspace), _stream(stream, workspace.device))
    if st:
        raise GdnError(st, "gdn_prefill_status")


@_on_stream
def gdn_prefill_fwd(q, k, v, alpha, beta, initial_state=None, final_state=None, y=None,
                    scale=1.0, return_final_state=True, workspace=None, stream=None):
    """Chunked prefill.  q, k [B, T, H, d_k]; v [B, T, H, d_v] (bf16 or fp32, one
    dtype); alpha, beta [B, T, H] fp32; initial_state [B, H, d_k, d_v] fp32 or
    None.  Returns (y [B, T, H, d_v] fp32, final_state or None).  ``final_state``
    may be ``initial_state`` for an in-place update.  ``workspace`` is a uint8
    device tensor of at least gdn_prefill_workspace_bytes(...) bytes; one is
    allocated when it is None."""
    lib = load_library()
    _require_gpu(q, "q")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _check(k, "k", (B, T, H, dk), q.dtype, dev)
    _check(v, "v", (B, T, H, dv), q.dtype, dev)
    _check(q, "q", (B, T, H, dk), q.dtype, dev)
    _check(alpha, "alpha", (B, T, H), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    _check(initial_state, "initial_state", (B, H, dk, dv), torch.float32, dev)
    if y is None:
        y = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _check(y, "y", (B, T, H, dv), torch.float32, dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check(final_state, "final_state", (B, H, dk, dv), torch.float32, dev)
    code = _dtype_code(q)
    need = int(lib.gdn_prefill_workspace_bytes(B, T, H, dk, dv, code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_prefill_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state),
                             _ptr(final_state), _ptr(y), B, T, H, dk, dv, code, float(scale),
                             _ptr(workspace), ws_bytes, _stream(stream, dev))
    if st:
        raise GdnError(st, "gdn_prefill_fwd")
    return y, final_state


def gdn_prefill_fwd_noalloc(q, k, v, alpha, beta, initial_state, final_state, y, scale=1.0, stream=None):
    """gdn_prefill_fwd whose scratch lives in the library's static per-GPU array
    (GDN_PREFILL_NOALLOC_SCRATCH_BYTES): neither this binding nor the library
    allocates anything, so the caller passes every output (``final_state``
    may be None, or ``initial_state`` for an in-place update).  Calls that can
    overlap on one GPU must not be issued (they share the array)."""
    lib = load_library()
    _require_gpu(q, "q")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _check(k, "k", (B, T, H, dk), q.dtype, dev)
    _check(v, "v", (B, T, H, dv), q.dtype, dev)
    _check(alpha, "alpha", (B, T, H), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    _check(initial_state, "initial_state", (B, H, dk, dv), torch.float32, dev)
    _check(final_state, "final_state", (B, H, dk, dv), torch.float32, dev)
    if y is None:
        raise ValueError("gdn_prefill_fwd_noalloc needs a preallocated y")
    _check(y, "y", (B, T, H, dv), torch.float32, dev)
    st = lib.gdn_prefill_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state),
                                     _ptr(final_state), _ptr(y), B, T, H, dk, dv, _dtype_code(q), float(scale),
                                     _stream(stream, dev))
    if st:
        raise GdnError(st, "gdn_prefill_fwd_noalloc")
    return y, final_state


@_on_stream
def gdn_decode_step(q, k, v, alpha, beta, state, y=None, scale=1.0, stream=None):
    """One decode step.  q, k [N, H, d_k]; v [N, H, d_v]; alpha, beta [N, H] fp32;
    state [N, H, d_k, d_v] fp32, updated in place.  Returns y [N, H, d_v] fp32."""
    lib = load_library()
    _require_gpu(q, "q")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _check(k, "k", (N, H, dk), q.dtype, dev)
    _check(v, "v", (N, H, dv), q.dtype, dev)
    _check(alpha, "alpha", (N, H), torch.float32, dev)
    _check(beta, "beta", (N, H), torch.float32, dev)
    _check(state, "state", (N, H, dk, dv), torch.float32, dev)
    if y is None:
        y = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    _check(y, "y", (N, H, dv), torch.float32, dev)
    st = lib.gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(y),
                             N, H, dk, dv, _dtype_code(q), float(scale), _stream(stream, dev))
    if st:
        raise GdnError(st, "gdn_decode_step")
    return y


@_on_stream
def gdn_gated_rmsnorm(y, z, weight=None, eps=1e-6, out=None, stream=None):
    """sigmoid(z) * RMSNorm(y) * (1 + weight) over the last axis.  y fp32, z bf16
    or fp32 of the same shape; weight [d_v] fp32 or None.  Returns out (z's dtype)."""
    lib = load_library()
    _require_gpu(y, "y")
    dv = y.shape[-1]
    dev = y.device
    _check(y, "y", y.shape, torch.float32, dev)
    _check(z, "z", y.shape, z.dtype, dev)
    _check(weight, "weight", (dv,), torch.float32, dev)
    if out is None:
        out = torch.empty(y.shape, dtype=z.dtype, device=dev)
    _check(out, "out", y.shape, z.dtype, dev)
    rows = y.numel() // dv if dv else 0
    st = lib.gdn_gated_rmsnorm(_ptr(y), _ptr(z), _ptr(weight), float(eps), _ptr(out), rows, dv,
                               _dtype_code(z), _stream(stream, dev))
    if st:
        raise GdnError(st, "gdn_gated_rmsnorm")
    return out


@_on_stream
def gdn_frontend_fwd(q_proj, k_proj, v_proj, conv_q, conv_k, conv_v, a_logit, b_logit, A, b_alpha,
                     q_hist=None, k_hist=None, v_hist=None, eps=1e-6, out=None, stream=None):
    """Front end: q, k = L2Norm(SiLU(ShortConv(proj))), v = SiLU(ShortConv(v_proj)),
    beta = sigmoid(b_logit), alpha = exp(-exp(A) softplus(a_logit + b_alpha)).
    q_proj, k_proj [B, T, H, d_k]; v_proj [B, T, H, d_v] (bf16 or fp32, one dtype);
    conv_* [H, d, W] fp32 (W <= 4); a_logit, b_logit [B, T, H] fp32; A, b_alpha [H]
    fp32; *_hist [B, W-1, H, d] or None.  ``out`` may be a tuple (q, k, v, alpha,
    beta) of preallocated tensors.  Returns (q, k, v, alpha, beta)."""
    lib = load_library()
    _require_gpu(q_proj, "q_proj")
    B, T, H, dk = q_proj.shape
    dv = v_proj.shape[-1]
    W = conv_q.shape[-1]
    dev, dt = q_proj.device, q_proj.dtype
    _check(k_proj, "k_proj", (B, T, H, dk), dt, dev)
    _check(v_proj, "v_proj", (B, T, H, dv), dt, dev)
    _check(conv_q, "conv_q", (H, dk, W), torch.float32, dev)
    _check(conv_k, "conv_k", (H, dk, W), torch.float32, dev)
    _check(conv_v, "conv_v", (H, dv, W), torch.float32, dev)
    _check(a_logit, "a_logit", (B, T, H), torch.float32, dev)
    _check(b_logit, "b_logit", (B, T, H), torch.float32, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(b_alpha, "b_alpha", (H,), torch.float32, dev)
    _check(q_hist, "q_hist", (B, W - 1, H, dk), dt, dev)
    _check(k_hist, "k_hist", (B, W - 1, H, dk), dt, dev)
    _check(v_hist, "v_hist", (B, W - 1, H, dv), dt, dev)
    if out is None:
        out = (torch.empty((B, T, H, dk), dtype=dt, device=dev), torch.empty((B, T, H, dk), dtype=dt, device=dev),
               torch.empty((B, T, H, dv), dtype=dt, device=dev),
               torch.empty((B, T, H), dtype=torch.float32, device=dev),
               torch.empty((B, T, H), dtype=torch.float32, device=dev))
    q, k, v, alpha, beta = out
    _check(q, "q", (B, T, H, dk), dt, dev)
    _check(k, "k", (B, T, H, dk), dt, dev)
    _check(v, "v", (B, T, H, dv), dt, dev)
    _check(alpha, "alpha", (B, T, H), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    st = lib.gdn_frontend_fwd(_ptr(q_proj), _ptr(k_proj), _ptr(v_proj), _ptr(conv_q), _ptr(conv_k), _ptr(conv_v),
                              _ptr(a_logit), _ptr(b_logit), _ptr(A), _ptr(b_alpha), _ptr(q_hist), _ptr(k_hist),
                              _ptr(v_hist), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), B, T, H, dk, dv, W,
                              _dtype_code(q_proj), float(eps), _stream(stream, dev))
    if st:
        raise GdnError(st, "gdn_frontend_fwd")
    return q, k, v, alpha, beta


@_on_stream
def gdn_decode_mtp_verify(q, k, v, alpha, beta, state, y=None, e=None, prefix_states=None, scale=1.0,
                          return_e=True, return_prefix_states=False, stream=None):
    """Verify a block of K draft tokens per sequence from the live states (read only).
    q, k [N, K, H, d_k]; v [N, K, H, d_v] (bf16 or fp32, one dtype); alpha, beta
    [N, K, H] fp32; state [N, H, d_k, d_v] fp32.  Returns (y [N, K, H, d_v],
    e [N, K, H, d_v] or None, prefix_states [N, K, H, d_k, d_v] or None), fp32."""
    lib = load_library()
    _require_gpu(q, "q")
    N, K, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _check(k, "k", (N, K, H, dk), q.dtype, dev)
    _check(v, "v", (N, K, H, dv), q.dtype, dev)
    _check(alpha, "alpha", (N, K, H), torch.float32, dev)
    _check(beta, "beta", (N, K, H), torch.float32, dev)
    _check(state, "state", (N, H, dk, dv), torch.float32, dev)
    if y is None:
        y = torch.empty((N, K, H, dv), dtype=torch.float32, device=dev)
    _check(y, "y", (N, K, H, dv), torch.float32, dev)
    if e is None and return_e:
        e = torch.empty((N, K, H, dv), dtype=torch.float32, device=dev)
    _check(e, "e", (N, K, H, dv), torch.float32, dev)
    if prefix_states is None and return_prefix_states:
        prefix_states = torch.empty((N, K, H, dk, dv), dtype=torch.float32, device=dev)
    _check(prefix_states, "prefix_states", (N, K, H, dk, dv), torch.float32, dev)
    st = lib.gdn_decode_mtp_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(y),
                                   _ptr(e), _ptr(prefix_states), N, K, H, dk, dv, _dtype_code(q), float(scale),
                                   _stream(stream, dev))
    if st:
        raise GdnError(st, "gdn_decode_mtp_verify")
    return y, e, prefix_states


@_on_stream
def gdn_decode_mtp_commit(k, alpha, beta, e, accepted, state, stream=None):
    """Advance each live state by its accepted drafts (int32 ``accepted`` [N] on the
    device, clamped to 0..K), using the misses ``e`` of gdn_decode_mtp_verify.
    k [N, K, H, d_k]; alpha, beta [N, K, H] fp32; e [N, K, H, d_v] fp32;
    state [N, H, d_k, d_v] fp32, updated in place.  Returns state."""
    lib = load_library()
    _require_gpu(k, "k")
    N, K, H, dk = k.shape
    dv = state.shape[-1]
    dev = k.device
    _check(alpha, "alpha", (N, K, H), torch.float32, dev)
    _check(beta, "beta", (N, K, H), torch.float32, dev)
    _check(e, "e", (N, K, H, dv), torch.float32, dev)
    _check(accepted, "accepted", (N,), torch.int32, dev)
    _check(state, "state", (N, H, dk, dv), torch.float32, dev)
    st = lib.gdn_decode_mtp_commit(_ptr(k), _ptr(alpha), _ptr(beta), _ptr(e), _ptr(accepted), _ptr(state),
                                   N, K, H, dk, dv, _dtype_code(k), _stream(stream, dev))
    if st:
        raise GdnError(st, "gdn_decode_mtp_commit")
    return state


def gdn_prefill_bwd_workspace_bytes(B, T, H, d_k, d_v, dtype):
    """Scratch bytes gdn_prefill_bwd needs (dtype: torch.bfloat16 or torch.float32)."""
    code = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(load_library().gdn_prefill_bwd_workspace_bytes(B, T, H, d_k, d_v, code))


@_on_stream
def gdn_prefill_bwd(q, k, v, alpha, beta, dy, initial_state=None, d_final_state=None, scale=1.0,
                    need_d_initial_state=True, workspace=None, out=None, stream=None):
    """Gradients of sum <dy, y> + <d_final_state, final_state> for gdn_prefill_fwd.
    q, k [B, T, H, d]; v [B, T, H, d] (bf16 or fp32, one dtype); alpha, beta
    [B, T, H] fp32; dy [B, T, H, d] fp32; initial_state, d_final_state
    [B, H, d, d] fp32 or None.  Returns (dq, dk, dv, dalpha, dbeta,
    d_initial_state or None), all fp32.  ``out`` may hold preallocated tensors
    in that order."""
    lib = load_library()
    _require_gpu(q, "q")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _check(k, "k", (B, T, H, dk), q.dtype, dev)
    _check(v, "v", (B, T, H, dv), q.dtype, dev)
    _check(q, "q", (B, T, H, dk), q.dtype, dev)
    _check(alpha, "alpha", (B, T, H), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    _check(dy, "dy", (B, T, H, dv), torch.float32, dev)
    _check(initial_state, "initial_state", (B, H, dk, dv), torch.float32, dev)
    _check(d_final_state, "d_final_state", (B, H, dk, dv), torch.float32, dev)
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = (torch.empty((B, T, H, dk), **f32), torch.empty((B, T, H, dk), **f32),
               torch.empty((B, T, H, dv), **f32), torch.empty((B, T, H), **f32), torch.empty((B, T, H), **f32),
               torch.empty((B, H, dk, dv), **f32) if need_d_initial_state else None)
    dq, dk_, dv_, da, db, dS0 = out
    _check(dq, "dq", (B, T, H, dk), torch.float32, dev)
    _check(dk_, "dk", (B, T, H, dk), torch.float32, dev)
    _check(dv_, "dv", (B, T, H, dv), torch.float32, dev)
    _check(da, "dalpha", (B, T, H), torch.float32, dev)
    _check(db, "dbeta", (B, T, H), torch.float32, dev)
    _check(dS0, "d_initial_state", (B, H, dk, dv), torch.float32, dev)
    code = _dtype_code(q)
    need = int(lib.gdn_prefill_bwd_workspace_bytes(B, T, H, dk, dv, code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_prefill_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(dy),
                             _ptr(d_final_state), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(da), _ptr(db), _ptr(dS0),
                             B, T, H, dk, dv, code, float(scale), _ptr(workspace), ws_bytes, _stream(stream, dev))
    if st:
        raise GdnError(st, "gdn_prefill_bwd")
    return dq, dk_, dv_, da, db, dS0


@_on_stream
def gdn_qsa_prep(q_proj, k_proj, r=4, rope_dims=64, rope_base=10000.0, eps=1e-6, q_weight=None, k_weight=None,
                 out=None, stream=None):
    """QSA indexer operands.  q_proj [B, n, H, D], k_proj [B, n, D] (bf16 or fp32, one
    dtype); q_weight, k_weight [D] fp32 or None.  Returns (q [B, n, H, D],
    kbar [B, n // r, D]) in the input dtype; ``out`` may hold both."""
    lib = load_library()
    _require_gpu(q_proj, "q_proj")
    B, n, H, D = q_proj.shape
    dev, dt = q_proj.device, q_proj.dtype
    _check(k_proj, "k_proj", (B, n, D), dt, dev)
    _check(q_weight, "q_weight", (D,), torch.float32, dev)
    _check(k_weight, "k_weight", (D,), torch.float32, dev)
    if out is None:
        out = (torch.empty((B, n, H, D), dtype=dt, device=dev), torch.empty((B, n // r, D), dtype=dt, device=dev))
    q, kbar = out
    _check(q, "q", (B, n, H, D), dt, dev)
    _check(kbar, "kbar", (B, n // r, D), dt, dev)
    st = lib.gdn_qsa_prep(_ptr(q_proj), _ptr(k_proj), _ptr(q_weight), _ptr(k_weight), _ptr(q), _ptr(kbar),
                          B, n, H, D, r, rope_dims, float(rope_base), float(eps), _dtype_code(q_proj),
                          _stream(stream, dev))
    if st:
        raise GdnError(st, "gdn_qsa_prep")
    return q, kbar


def gdn_qsa_select_workspace_bytes(B, n, H, D, r, K, dtype):
    code = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(load_library().gdn_qsa_select_workspace_bytes(B, n, H, D, r, K, code))


@_on_stream
def gdn_qsa_select(q, kbar, r=4, K=2048, block_idx=None, workspace=None, stream=None):
    """Top-ceil(K / r) complete key blocks per query.  q [B, n, H, D], kbar
    [B, n // r, D] (bf16 or fp32).  Returns block_idx [B, n, ceil(K / r)] int32,
    ascending, -1 padded."""
    lib = load_library()
    _require_gpu(q, "q")
    B, n, H, D = q.shape
    dev = q.device
    KB = -(-K // r)
    _check(kbar, "kbar", (B, n // r, D), q.dtype, dev)
    if block_idx is None:
        block_idx = torch.empty((B, n, KB), dtype=torch.int32, device=dev)
    _check(block_idx, "block_idx", (B, n, KB), torch.int32, dev)
    code = _dtype_code(q)
    need = int(lib.gdn_qsa_select_workspace_bytes(B, n, H, D, r, K, code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_qsa_select(_ptr(q), _ptr(kbar), _ptr(block_idx), B, n, H, D, r, K, code, _ptr(workspace),
                            ws_bytes, _stream(stream, dev))
    if st:
        raise GdnError(st, "gdn_qsa_select")
    return block_idx


@_on_stream
def gdn_decode_mtp_commit_verify(q, k, v, alpha, beta, state, prev_k, prev_alpha, prev_beta, prev_e,
                                 prev_accepted, y=None, e=None, scale=1.0, return_e=True, stream=None):
    """Commit the previous block's accepted drafts onto ``state`` (in place) and
    verify the new block from the committed state, in one pass over the state.
    New block: q, k [N, K, H, d_k]; v [N, K, H, d_v]; alpha, beta [N, K, H].
    Previous block: prev_k [N, K_prev, H, d_k]; prev_alpha, prev_beta
    [N, K_prev, H]; prev_e [N, K_prev, H, d_v]; prev_accepted [N] int32.
    Returns (y, e) of the new block."""
    lib = load_library()
    _require_gpu(q, "q")
    N, K, H, dk = q.shape
    dv = v.shape[-1]
    Kp = prev_k.shape[1]
    dev = q.device
    _check(k, "k", (N, K, H, dk), q.dtype, dev)
    _check(v, "v", (N, K, H, dv), q.dtype, dev)
    _check(alpha, "alpha", (N, K, H), torch.float32, dev)
    _check(beta, "beta", (N, K, H), torch.float32, dev)
    _check(state, "state", (N, H, dk, dv), torch.float32, dev)
    _check(prev_k, "prev_k", (N, Kp, H, dk), q.dtype, dev)
    _check(prev_alpha, "prev_alpha", (N, Kp, H), torch.float32, dev)
    _check(prev_beta, "prev_beta", (N, Kp, H), torch.float32, dev)
    _check(prev_e, "prev_e", (N, Kp, H, dv), torch.float32, dev)
    _check(prev_accepted, "prev_accepted", (N,), torch.int32, dev)
    if y is None:
        y = torch.empty((N, K, H, dv), dtype=torch.float32, device=dev)
    _check(y, "y", (N, K, H, dv), torch.float32, dev)
    if e is None and return_e:
        e = torch.empty((N, K, H, dv), dtype=torch.float32, device=dev)
    _check(e, "e", (N, K, H, dv), torch.float32, dev)
    st = lib.gdn_decode_mtp_commit_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(y),
                                          _ptr(e), _ptr(prev_k), _ptr(prev_alpha), _ptr(prev_beta), _ptr(prev_e),
                                          _ptr(prev_accepted), N, K, Kp, H, dk, dv, _dtype_code(q), float(scale),
                                          _stream(stream, dev))
    if st:
        raise GdnError(st, "gdn_decode_mtp_commit_verify")
    return y, e
