"""GPU-side checks of the chunk algebra of the bf16 prefill, below the level of
y and the final state:

* the chunk-parallel pass's workspace (a caller-provided device buffer) holds,
  per (head, chunk), T' = (I + A)^-1 diag(beta) with
  A_ti = beta_t Gamma_ti k_t.k_i (i < t), and the base-2 gates
  g2 = sum of log2 alpha, gamma = 2^g2, d = 2^(g2_last - g2),
  w = 2^(g2_blockend - g2); they are compared with the same quantities
  computed here in float64 from the inputs (slinene page, Module A, and the
  chunkwise form of its delta rule);
* the states at chunk boundaries: a call over the first 64 m tokens ends in
  the oracle's state at t = 64 m.

The workspace layout read here is the library's documented one: a 256-byte
status header, then per (b * H + h, chunk) six 16 x 32 fp16 tiles of T' with
their columns in split-K order followed by the four float32 gate arrays.
"""

import numpy as np
import pytest
import torch

from oracle import gated_delta_recurrence
from tests.gpu_util import TOL, check, dev, host, prefill, say
from workloads import prefill_inputs
import linear_attention_recurrence_rule_amd as gdn

pytestmark = pytest.mark.gpu

C = 64
LOG2_FLOOR = -30.0 / np.log(2.0)          # the kernels' floor of log alpha, in base 2
TILES = [(0, 0), (1, 0), (2, 0), (2, 1), (3, 0), (3, 1)]
WS_HALFS = 6 * 512 + 2 * 4 * C            # halfs per (head, chunk)


def _split_cols(h):
    """Chunk columns held by positions 0 .. 31 of a tile of column group h."""
    pos = np.arange(32)
    g, s = pos // 8, pos % 8
    return 32 * h + 16 * (s // 4) + 4 * g + s % 4


def _tprime_from_tiles(halfs):
    Tp = np.zeros((C, C))
    for t, (I, h) in enumerate(TILES):
        tile = halfs[t * 512:(t + 1) * 512].astype(np.float64).reshape(16, 32)
        Tp[16 * I:16 * I + 16, _split_cols(h)] = tile
    return Tp


def _reference(k, alpha, beta, T, c):
    """float64 T' and gates of chunk c of one head (rows past T: alpha = 1, beta = 0)."""
    t = np.arange(c * C, (c + 1) * C)
    live = t < T
    a = np.where(live, alpha[np.minimum(t, T - 1)], 1.0)
    be = np.where(live, beta[np.minimum(t, T - 1)], 0.0)
    K = k[np.minimum(t, T - 1)].astype(np.float64)
    with np.errstate(divide="ignore"):
        g2 = np.cumsum(np.maximum(np.log2(a), LOG2_FLOOR))
    Gam = np.where(np.tril(np.ones((C, C), bool)), np.exp2(g2[:, None] - g2[None, :]), 0.0)
    A = np.tril(be[:, None] * Gam * (K @ K.T), -1)
    Tp = np.linalg.inv(np.eye(C) + A) * be[None, :]
    blockend = g2[(np.arange(C) | 15)]
    gates = np.stack([g2, np.exp2(g2), np.exp2(g2[-1] - g2), np.exp2(blockend - g2)])
    return Tp, gates


@pytest.mark.parametrize("dk", [64, 128])
def test_workspace_holds_chunk_inverse_and_gates(dk):
    """T' of every (head, chunk), ragged last chunk included, and the gates."""
    say(f"chunk algebra: workspace T' and gates, d_k = {dk}")
    B, T, H = 1, 200, 3
    d = prefill_inputs(B, T, H, dk, dk, "bf16", -1.0, 0.5, seed=31)
    need = gdn.gdn_prefill_workspace_bytes(B, T, H, dk, dk, torch.bfloat16)
    nch = (T + C - 1) // C
    assert need == 256 + B * H * nch * WS_HALFS * 2
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    prefill(*(dev(d[x], "bf16") for x in ("q", "k", "v")), dev(d["alpha"]), dev(d["beta"]), workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()[256:]
    worst_t, worst_g = 0.0, 0.0
    for h in range(H):
        for c in range(nch):
            slot = raw[((h * nch) + c) * WS_HALFS * 2:((h * nch) + c + 1) * WS_HALFS * 2]
            halfs = slot[:6 * 512 * 2].view(np.float16)
            gates = slot[6 * 512 * 2:].view(np.float32).reshape(4, C).astype(np.float64)
            Tp_ref, g_ref = _reference(d["k"][0, :, h], d["alpha"][0, :, h], d["beta"][0, :, h], T, c)
            Tp = _tprime_from_tiles(halfs)
            # T' is stored in fp16 after fp16-operand block products in float32:
            # a few fp16 roundings of entries of size <= max|T'|
            et = np.max(np.abs(Tp - Tp_ref)) / np.max(np.abs(Tp_ref))
            worst_t = max(worst_t, et)
            assert et <= 4e-3, f"head {h} chunk {c}: T' error {et:.3e}"
            assert np.all(Tp[np.triu_indices(C, 1)] == 0), "T' not lower triangular"
            # gates: a float32 prefix sum of 64 log2 terms, then native 2^x
            eg = np.max(np.abs(gates[0] - g_ref[0])) / max(1.0, np.max(np.abs(g_ref[0])))
            ef = max(np.max(np.abs(gates[i] - g_ref[i]) / np.maximum(np.abs(g_ref[i]), 1e-30)) for i in (1, 2, 3))
            worst_g = max(worst_g, eg, ef)
            assert eg <= 2e-5 and ef <= 2e-4, f"head {h} chunk {c}: gate errors {eg:.3e} {ef:.3e}"
    say(f"    worst T' error {worst_t:.3e}, worst gate error {worst_g:.3e}")


def test_states_at_chunk_boundaries():
    """A call over the first 64 m tokens ends in the oracle's state after token
    64 m (the state the sequential walk carries into chunk m)."""
    say("chunk algebra: states at chunk boundaries")
    B, T, H, D = 2, 320, 2, 128
    d = prefill_inputs(B, T, H, D, D, "bf16", -1.0, 0.5, seed=32, state_std=0.1)
    for m in (1, 2, 3, 5):
        t = 64 * m
        sl = {x: d[x][:, :t] for x in ("q", "k", "v", "alpha", "beta")}
        _, S = prefill(*(dev(sl[x], "bf16") for x in ("q", "k", "v")), dev(sl["alpha"]), dev(sl["beta"]),
                       dev(d["initial_state"]))
        _, S_ref = gated_delta_recurrence(sl["q"], sl["k"], sl["v"], sl["alpha"], sl["beta"], d["initial_state"])
        check(f"state after token {t}", host(S), S_ref, TOL["bf16"])
