"""C ABI checks that need no GPU: the library loads, exports every entry point
include/gdn.h declares, and rejects bad arguments with the documented status
codes before anything is launched (every call below fails validation, so no
HIP call is made)."""

import ctypes
import os
import re
import subprocess

import pytest

import linear_attention_recurrence_rule_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_LAUNCH, ERR_WORKSPACE, ERR_DEVICE = range(9)
FAKE = 0x10000          # an aligned, never-dereferenced address
MISALIGNED = 0x10004


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:gdn_status|const char\*|size_t)\s+(gdn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["gdn_decode_mtp_commit", "gdn_decode_mtp_commit_verify",
                                    "gdn_decode_mtp_verify", "gdn_decode_step",
                                    "gdn_frontend_fwd", "gdn_gated_rmsnorm", "gdn_prefill_bwd",
                                    "gdn_prefill_bwd_workspace_bytes", "gdn_prefill_fwd",
                                    "gdn_prefill_fwd_noalloc", "gdn_prefill_status",
                                    "gdn_prefill_workspace_bytes", "gdn_qsa_prep", "gdn_qsa_select",
                                    "gdn_qsa_select_workspace_bytes", "gdn_status_string"]


def test_library_exports_every_declared_symbol():
    lib = gdn.load_library()
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdn_\w+)", out))
    for name in declared_functions():
        assert name in exported
        assert hasattr(lib, name)


def test_status_strings():
    assert gdn.gdn_status_string(OK) == "ok"
    for s in range(1, 9):
        assert gdn.gdn_status_string(s) and gdn.gdn_status_string(s) != "unknown status"
    assert gdn.gdn_status_string(99) == "unknown status"


def _prefill(q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s0=None, sT=FAKE, y=FAKE,
             B=1, T=8, H=2, dk=64, dv=64, dtype=1, ws=FAKE, ws_bytes=1 << 30):
    lib = gdn.load_library()
    return lib.gdn_prefill_fwd(q, k, v, a, b, s0, sT, y, B, T, H, dk, dv, dtype, 1.0, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=2), ERR_DTYPE),
    (dict(dtype=-1), ERR_DTYPE),
    (dict(B=0), ERR_SHAPE),
    (dict(H=0), ERR_SHAPE),
    (dict(T=-1), ERR_SHAPE),
    (dict(dk=48), ERR_UNSUPPORTED),
    (dict(dv=256), ERR_UNSUPPORTED),
    (dict(dk=8), ERR_UNSUPPORTED),
    (dict(B=1 << 20, T=1 << 20, H=1 << 10), ERR_UNSUPPORTED),
    (dict(q=None), ERR_NULL),
    (dict(y=None), ERR_NULL),
    (dict(a=None), ERR_NULL),
    (dict(v=MISALIGNED), ERR_ALIGN),
    (dict(s0=MISALIGNED), ERR_ALIGN),
    (dict(sT=MISALIGNED), ERR_ALIGN),
    (dict(ws=MISALIGNED), ERR_ALIGN),
    (dict(B=300, H=300), ERR_UNSUPPORTED),
    (dict(ws=None), ERR_WORKSPACE),
    (dict(ws_bytes=5119 + 256), ERR_WORKSPACE),
])
def test_prefill_rejects(kwargs, status):
    assert _prefill(**kwargs) == status


def test_workspace_bytes():
    lib = gdn.load_library()
    # bf16: a 256-byte status header, then per (sequence, head, 64-token
    # chunk) the 10 lower fp16 16x16 blocks of T' (5120 bytes) and four
    # float32 gate vectors of 64 (1024 bytes)
    per_chunk = 6 * 512 * 2 + 4 * 64 * 4
    assert lib.gdn_prefill_workspace_bytes(1, 8, 2, 64, 64, 1) == 256 + 2 * per_chunk
    assert lib.gdn_prefill_workspace_bytes(2, 65, 3, 128, 128, 1) == 256 + 2 * 3 * 2 * per_chunk
    assert lib.gdn_prefill_workspace_bytes(2, 65, 3, 128, 128, 0) == 0
    assert lib.gdn_prefill_workspace_bytes(2, 0, 3, 128, 128, 1) == 0
    assert lib.gdn_prefill_workspace_bytes(2, 65, 3, 48, 128, 1) == 0


def _prefill_noalloc(q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s0=None, sT=FAKE, y=FAKE,
                     B=1, T=8, H=2, dk=64, dv=64, dtype=1):
    lib = gdn.load_library()
    lib.gdn_prefill_fwd_noalloc.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 6 + [ctypes.c_float,
                                                                                         ctypes.c_void_p]
    return lib.gdn_prefill_fwd_noalloc(q, k, v, a, b, s0, sT, y, B, T, H, dk, dv, dtype, 1.0, None)


def test_prefill_noalloc_rejects_sizes_beyond_its_scratch():
    lib = gdn.load_library()
    limit = 128 << 20
    # 18724 (sequence, head, chunk) units fit the 128 MiB array, 18725 do not
    assert lib.gdn_prefill_workspace_bytes(1, 18724 * 64, 1, 128, 128, 1) <= limit
    assert lib.gdn_prefill_workspace_bytes(1, 18725 * 64, 1, 128, 128, 1) > limit
    assert _prefill_noalloc(B=1, T=18725 * 64, H=1, dk=128, dv=128) == ERR_WORKSPACE
    assert _prefill_noalloc(B=4, T=32768, H=32, dk=128, dv=128) == ERR_WORKSPACE
    # argument errors are reported as by gdn_prefill_fwd (checked before anything else)
    assert _prefill_noalloc(dtype=2) == ERR_DTYPE
    assert _prefill_noalloc(dk=48) == ERR_UNSUPPORTED
    assert _prefill_noalloc(q=None) == ERR_NULL
    assert _prefill_noalloc(y=MISALIGNED) == ERR_ALIGN


def test_prefill_status_rejects_bad_pointers():
    lib = gdn.load_library()
    lib.gdn_prefill_status.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert lib.gdn_prefill_status(None, None) == ERR_NULL
    assert lib.gdn_prefill_status(MISALIGNED, None) == ERR_ALIGN


def test_prefill_empty_without_state_is_a_no_op():
    assert _prefill(q=None, k=None, v=None, a=None, b=None, y=None, sT=None, T=0, ws=None) == OK


def _decode(q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s=FAKE, y=FAKE, N=4, H=2, dk=128, dv=128, dtype=1):
    lib = gdn.load_library()
    return lib.gdn_decode_step(q, k, v, a, b, s, y, N, H, dk, dv, dtype, 1.0, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=5), ERR_DTYPE),
    (dict(N=-1), ERR_SHAPE),
    (dict(H=0), ERR_SHAPE),
    (dict(dk=100), ERR_UNSUPPORTED),
    (dict(s=None), ERR_NULL),
    (dict(k=None), ERR_NULL),
    (dict(y=MISALIGNED), ERR_ALIGN),
    (dict(s=MISALIGNED), ERR_ALIGN),
])
def test_decode_rejects(kwargs, status):
    assert _decode(**kwargs) == status


def test_decode_zero_sequences_is_a_no_op():
    assert _decode(q=None, s=None, N=0) == OK


def _norm(y=FAKE, z=FAKE, w=None, out=FAKE, rows=16, dv=128, dtype=1):
    lib = gdn.load_library()
    return lib.gdn_gated_rmsnorm(y, z, w, ctypes.c_float(1e-6), out, rows, dv, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=3), ERR_DTYPE),
    (dict(rows=-2), ERR_SHAPE),
    (dict(dv=96), ERR_UNSUPPORTED),
    (dict(z=None), ERR_NULL),
    (dict(out=None), ERR_NULL),
    (dict(w=MISALIGNED), ERR_ALIGN),
    (dict(y=MISALIGNED), ERR_ALIGN),
])
def test_norm_rejects(kwargs, status):
    assert _norm(**kwargs) == status


def test_norm_zero_rows_is_a_no_op():
    assert _norm(y=None, z=None, out=None, rows=0) == OK


def test_python_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 4, 2, 16)
    a = torch.zeros(1, 4, 2)
    with pytest.raises(ValueError, match="GPU tensor"):
        gdn.gdn_prefill_fwd(q, q, q, a, a)
    with pytest.raises(ValueError, match="GPU tensor"):
        gdn.gdn_decode_step(q[0], q[0], q[0], a[0], a[0], torch.zeros(4, 2, 16, 16))
    with pytest.raises(ValueError, match="GPU tensor"):
        gdn.gdn_gated_rmsnorm(q, q)


def _frontend(qp=FAKE, kp=FAKE, vp=FAKE, cq=FAKE, ck=FAKE, cv=FAKE, al=FAKE, bl=FAKE, A=FAKE, ba=FAKE,
              qh=None, kh=None, vh=None, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE,
              B=1, T=8, H=2, dk=64, dv=64, W=4, dtype=1, eps=1e-6):
    lib = gdn.load_library()
    return lib.gdn_frontend_fwd(qp, kp, vp, cq, ck, cv, al, bl, A, ba, qh, kh, vh, q, k, v, a, b,
                                B, T, H, dk, dv, W, dtype, eps, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=3), ERR_DTYPE),
    (dict(B=0), ERR_SHAPE),
    (dict(T=-2), ERR_SHAPE),
    (dict(W=0), ERR_SHAPE),
    (dict(eps=-1.0), ERR_SHAPE),
    (dict(eps=float("nan")), ERR_SHAPE),
    (dict(W=5), ERR_UNSUPPORTED),
    (dict(dk=96), ERR_UNSUPPORTED),
    (dict(qp=None), ERR_NULL),
    (dict(cv=None), ERR_NULL),
    (dict(A=None), ERR_NULL),
    (dict(b=None), ERR_NULL),
    (dict(kp=MISALIGNED), ERR_ALIGN),
    (dict(vh=MISALIGNED), ERR_ALIGN),
    (dict(v=MISALIGNED), ERR_ALIGN),
])
def test_frontend_rejects(kwargs, status):
    assert _frontend(**kwargs) == status


def test_frontend_empty_sequence_is_a_no_op():
    assert _frontend(T=0, qp=None, q=None) == OK


def _verify(q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s=FAKE, y=FAKE, e=None, p=None,
            N=4, K=4, H=2, dk=128, dv=128, dtype=1):
    lib = gdn.load_library()
    return lib.gdn_decode_mtp_verify(q, k, v, a, b, s, y, e, p, N, K, H, dk, dv, dtype, 1.0, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=4), ERR_DTYPE),
    (dict(N=-1), ERR_SHAPE),
    (dict(K=-1), ERR_SHAPE),
    (dict(H=0), ERR_SHAPE),
    (dict(K=9), ERR_UNSUPPORTED),
    (dict(dv=48), ERR_UNSUPPORTED),
    (dict(q=None), ERR_NULL),
    (dict(s=None), ERR_NULL),
    (dict(y=None), ERR_NULL),
    (dict(e=MISALIGNED), ERR_ALIGN),
    (dict(p=MISALIGNED), ERR_ALIGN),
    (dict(s=MISALIGNED), ERR_ALIGN),
])
def test_mtp_verify_rejects(kwargs, status):
    assert _verify(**kwargs) == status


def test_mtp_verify_empty_is_a_no_op():
    assert _verify(N=0, q=None) == OK
    assert _verify(K=0, q=None) == OK


def _commit(k=FAKE, a=FAKE, b=FAKE, e=FAKE, acc=FAKE, s=FAKE, N=4, K=4, H=2, dk=128, dv=128, dtype=1):
    lib = gdn.load_library()
    return lib.gdn_decode_mtp_commit(k, a, b, e, acc, s, N, K, H, dk, dv, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=2), ERR_DTYPE),
    (dict(N=-3), ERR_SHAPE),
    (dict(K=-1), ERR_SHAPE),
    (dict(K=12), ERR_UNSUPPORTED),
    (dict(dk=8), ERR_UNSUPPORTED),
    (dict(acc=None), ERR_NULL),
    (dict(e=None), ERR_NULL),
    (dict(s=None), ERR_NULL),
    (dict(e=MISALIGNED), ERR_ALIGN),
    (dict(s=MISALIGNED), ERR_ALIGN),
])
def test_mtp_commit_rejects(kwargs, status):
    assert _commit(**kwargs) == status


def test_mtp_commit_empty_is_a_no_op():
    assert _commit(N=0, s=None) == OK
    assert _commit(K=0, s=None) == OK


def _bwd(q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s0=None, dy=FAKE, dsT=None, dq=FAKE, dk=FAKE, dv=FAKE,
         da=FAKE, db=FAKE, ds0=None, B=1, T=8, H=2, d_k=64, d_v=64, dtype=1, ws=FAKE, ws_bytes=1 << 40):
    lib = gdn.load_library()
    return lib.gdn_prefill_bwd(q, k, v, a, b, s0, dy, dsT, dq, dk, dv, da, db, ds0, B, T, H, d_k, d_v, dtype,
                               1.0, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=2), ERR_DTYPE),
    (dict(B=0), ERR_SHAPE),
    (dict(T=-1), ERR_SHAPE),
    (dict(d_k=64, d_v=128), ERR_UNSUPPORTED),
    (dict(d_k=48, d_v=48), ERR_UNSUPPORTED),
    (dict(H=70000), ERR_UNSUPPORTED),
    (dict(dy=None), ERR_NULL),
    (dict(db=None), ERR_NULL),
    (dict(ws=None), ERR_WORKSPACE),
    (dict(ws_bytes=16), ERR_WORKSPACE),
    (dict(dq=MISALIGNED), ERR_ALIGN),
    (dict(ds0=MISALIGNED), ERR_ALIGN),
    (dict(ws=MISALIGNED), ERR_ALIGN),
])
def test_bwd_rejects(kwargs, status):
    assert _bwd(**kwargs) == status


def test_bwd_workspace_bytes():
    lib = gdn.load_library()
    n = lib.gdn_prefill_bwd_workspace_bytes(1, 100, 2, 64, 64, 1)
    # two chunks x two heads: g, T, P, M, S, dS', E, dR in float32
    per = 64 * 4 + 3 * 64 * 64 * 4 + 2 * 64 * 64 * 4 + 2 * 64 * 64 * 4
    assert n >= 4 * per
    assert n < 4 * per + 8 * 256
    assert lib.gdn_prefill_bwd_workspace_bytes(1, 0, 2, 64, 64, 1) == 0
    assert lib.gdn_prefill_bwd_workspace_bytes(1, 100, 2, 64, 32, 1) == 0


def test_bwd_empty_sequence_without_state_gradient_is_a_no_op():
    assert _bwd(T=0, q=None, dy=None, dq=None, ws=None, ws_bytes=0) == OK


def _qprep(qp=FAKE, kp=FAKE, qw=None, kw=None, qo=FAKE, ko=FAKE, B=1, n=64, H=4, D=128, r=4, R=64,
           base=10000.0, eps=1e-6, dtype=1):
    lib = gdn.load_library()
    return lib.gdn_qsa_prep(qp, kp, qw, kw, qo, ko, B, n, H, D, r, R, base, eps, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=5), ERR_DTYPE),
    (dict(B=0), ERR_SHAPE),
    (dict(n=-1), ERR_SHAPE),
    (dict(r=0), ERR_SHAPE),
    (dict(R=3), ERR_SHAPE),
    (dict(eps=-1.0), ERR_SHAPE),
    (dict(base=0.0), ERR_SHAPE),
    (dict(D=96), ERR_UNSUPPORTED),
    (dict(D=32, R=64), ERR_UNSUPPORTED),
    (dict(kp=None), ERR_NULL),
    (dict(ko=None), ERR_NULL),
    (dict(qw=MISALIGNED), ERR_ALIGN),
    (dict(qo=MISALIGNED), ERR_ALIGN),
])
def test_qsa_prep_rejects(kwargs, status):
    assert _qprep(**kwargs) == status


def test_qsa_prep_empty_is_a_no_op():
    assert _qprep(n=0, qp=None, kp=None) == OK


def _qsel(q=FAKE, kb=FAKE, idx=FAKE, B=1, n=64, H=4, D=128, r=4, K=16, dtype=1, ws=FAKE, ws_bytes=1 << 40):
    lib = gdn.load_library()
    return lib.gdn_qsa_select(q, kb, idx, B, n, H, D, r, K, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=2), ERR_DTYPE),
    (dict(H=0), ERR_SHAPE),
    (dict(K=0), ERR_SHAPE),
    (dict(r=0), ERR_SHAPE),
    (dict(D=48), ERR_UNSUPPORTED),
    (dict(q=None), ERR_NULL),
    (dict(idx=None), ERR_NULL),
    (dict(kb=None), ERR_NULL),
    (dict(ws=None), ERR_WORKSPACE),
    (dict(ws_bytes=4), ERR_WORKSPACE),
    (dict(idx=MISALIGNED), ERR_ALIGN),
    (dict(ws=MISALIGNED), ERR_ALIGN),
])
def test_qsa_select_rejects(kwargs, status):
    assert _qsel(**kwargs) == status


def test_qsa_select_workspace_bytes():
    lib = gdn.load_library()
    up = lambda x: (x + 255) // 256 * 256
    # four query heads, n = 100 tokens, r = 4 (25 blocks), K = 2048 (K_B = 512),
    # 200 query rows: key maxima + queue count, per-row band (8 B), 16 sub-list
    # lengths (4 B each), the queue (4 B), 16 sub-lists of
    # 512 / 16 + 1024 / 16 + 32 (bits, block) pairs (8 B) per row, and 512
    # scratch rows of 64 floats
    rows = 2 * 100
    four = (up(2 * 4) + 256 + up(rows * 8) + up(rows * 16 * 4) + up(rows * 4) + up(rows * 16 * 128 * 8)
            + up(256 * 64 * 4))
    assert lib.gdn_qsa_select_workspace_bytes(2, 100, 4, 128, 4, 2048, 1) == four
    # other head counts store the fp32 scores, rows padded to 64 blocks
    assert lib.gdn_qsa_select_workspace_bytes(2, 100, 2, 128, 4, 2048, 1) == 2 * 100 * 64 * 4
    assert lib.gdn_qsa_select_workspace_bytes(2, 100, 4, 100, 4, 2048, 1) == 0


def test_qsa_select_empty_is_a_no_op():
    assert _qsel(n=0, q=None, idx=None, ws=None, ws_bytes=0) == OK


def _cv(q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s=FAKE, y=FAKE, e=None, pk=FAKE, pa=FAKE, pb=FAKE, pe=FAKE,
        pacc=FAKE, N=4, K=4, Kp=4, H=2, dk=128, dv=128, dtype=1):
    lib = gdn.load_library()
    return lib.gdn_decode_mtp_commit_verify(q, k, v, a, b, s, y, e, pk, pa, pb, pe, pacc, N, K, Kp, H, dk, dv,
                                            dtype, 1.0, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=3), ERR_DTYPE),
    (dict(K=0), ERR_SHAPE),
    (dict(Kp=0), ERR_SHAPE),
    (dict(N=-1), ERR_SHAPE),
    (dict(Kp=9), ERR_UNSUPPORTED),
    (dict(dk=24), ERR_UNSUPPORTED),
    (dict(pe=None), ERR_NULL),
    (dict(pacc=None), ERR_NULL),
    (dict(s=None), ERR_NULL),
    (dict(pk=MISALIGNED), ERR_ALIGN),
    (dict(e=MISALIGNED), ERR_ALIGN),
    (dict(e=FAKE, pe=FAKE, K=4, Kp=3), ERR_SHAPE),   # e aliasing prev_e needs K == K_prev
])
def test_mtp_commit_verify_rejects(kwargs, status):
    assert _cv(**kwargs) == status


def test_mtp_commit_verify_empty_is_a_no_op():
    assert _cv(N=0, q=None, s=None) == OK
