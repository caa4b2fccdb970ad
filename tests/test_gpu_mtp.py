"""gdn_decode_mtp_verify / gdn_decode_mtp_commit on the GPU against the float64
multi-token decode oracle (oracle/mtp_ref.py) and the plain recurrence."""

import numpy as np
import pytest
import torch

from oracle import gated_delta_recurrence, mtp_commit, mtp_verify
from tests.gpu_util import check, dev, host, say
from workloads import decode_initial_state, mtp_draft_inputs, prefill_inputs
import linear_attention_recurrence_rule_amd as gdn

pytestmark = pytest.mark.gpu

# float32 arithmetic on exact inputs: K-term recurrences over d_k-term dot
# products; errors stay near 1e-6 of the rms, the float32 bound is used for
# both input dtypes (as for the single-token decode step).
MTP_TOL = 1e-4


def _block(N, K, H, dk, dv, dtype, seed, state_std=0.3):
    d = prefill_inputs(N, K, H, dk, dv, dtype, -1.0, 0.5, seed=seed)
    rng = np.random.default_rng([seed, 99])
    S0 = (state_std * rng.standard_normal((N, H, dk, dv))).astype(np.float32)
    return d, S0


def _gpu_block(d, dtype):
    return (dev(d["q"], dtype), dev(d["k"], dtype), dev(d["v"], dtype), dev(d["alpha"]), dev(d["beta"]))


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 3, 4, 5, 8])
def test_verify_and_commit_small(dk, dv, dtype, K):
    say(f"mtp small dk={dk} dv={dv} {dtype} K={K}")
    N, H = 5, 3
    d, S0 = _block(N, K, H, dk, dv, dtype, seed=dk + 7 * dv + 31 * K)
    q, k, v, a, b = _gpu_block(d, dtype)
    state = dev(S0)
    y, e, pref = gdn.gdn_decode_mtp_verify(q, k, v, a, b, state, scale=0.8, return_prefix_states=True)
    y_ref, e_ref, p_ref = mtp_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S0, scale=0.8)
    check("y", host(y), y_ref, MTP_TOL)
    check("e", host(e), e_ref, MTP_TOL)
    check("prefix states", host(pref), p_ref, MTP_TOL)
    np.testing.assert_array_equal(host(state), S0.astype(np.float64))      # verify leaves it alone
    accepted = np.array([0, K, 1, (K + 1) // 2, K - 1][:N], dtype=np.int32)
    gdn.gdn_decode_mtp_commit(k, a, b, e, torch.from_numpy(accepted).cuda(), state)
    S_ref = mtp_commit(d["k"], d["alpha"], d["beta"], e_ref, accepted, S0)
    check("committed state", host(state), S_ref, MTP_TOL)
    np.testing.assert_array_equal(host(state)[0], S0[0].astype(np.float64))  # accepted 0: untouched


def test_commit_clamps_out_of_range_counts():
    say("mtp commit clamps")
    N, K, H, dk, dv = 4, 4, 2, 64, 64
    d, S0 = _block(N, K, H, dk, dv, "bf16", seed=5)
    q, k, v, a, b = _gpu_block(d, "bf16")
    state = dev(S0)
    _, e, _ = gdn.gdn_decode_mtp_verify(q, k, v, a, b, state)
    raw = np.array([-3, 9, 2, 4], dtype=np.int32)
    gdn.gdn_decode_mtp_commit(k, a, b, e, torch.from_numpy(raw).cuda(), state)
    _, e_ref, _ = mtp_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S0)
    S_ref = mtp_commit(d["k"], d["alpha"], d["beta"], e_ref, np.clip(raw, 0, K), S0)
    check("state", host(state), S_ref, MTP_TOL)


def test_one_token_block_equals_decode_step():
    """K = 1 verify + commit(1) is one gdn_decode_step (GPU against GPU and oracle)."""
    say("mtp K=1 vs decode step")
    N, H, d_ = 6, 4, 128
    d, S0 = _block(N, 1, H, d_, d_, "bf16", seed=11)
    q, k, v, a, b = _gpu_block(d, "bf16")
    s_mtp, s_dec = dev(S0), dev(S0)
    y_mtp, e, _ = gdn.gdn_decode_mtp_verify(q, k, v, a, b, s_mtp)
    gdn.gdn_decode_mtp_commit(k, a, b, e, torch.ones(N, dtype=torch.int32, device="cuda"), s_mtp)
    y_dec = gdn.gdn_decode_step(q[:, 0], k[:, 0], v[:, 0], a[:, 0], b[:, 0], s_dec)
    y_ref, S_ref = gated_delta_recurrence(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S0)
    check("y vs oracle", host(y_mtp)[:, 0], y_ref[:, 0], MTP_TOL)
    check("y vs decode step", host(y_mtp)[:, 0], host(y_dec), MTP_TOL)
    check("state vs oracle", host(s_mtp), S_ref, MTP_TOL)
    check("state vs decode step", host(s_mtp), host(s_dec), MTP_TOL)


def test_rounds_of_drafts_follow_the_accepted_tokens():
    """Several verify/commit rounds with random acceptance: the outputs of the
    accepted drafts and the final state equal one plain recurrence over the
    accepted tokens only (rejected drafts leave no trace)."""
    say("mtp rounds")
    N, K, H, d_ = 4, 4, 3, 64
    rng = np.random.default_rng(21)
    S0 = (0.2 * rng.standard_normal((N, H, d_, d_))).astype(np.float32)
    state = dev(S0)
    kept = [{x: [] for x in ("q", "k", "v", "alpha", "beta", "y")} for _ in range(N)]
    for rnd in range(6):
        d = prefill_inputs(N, K, H, d_, d_, "bf16", -1.0, 0.5, seed=[21, rnd])
        q, k, v, a, b = _gpu_block(d, "bf16")
        y, e, _ = gdn.gdn_decode_mtp_verify(q, k, v, a, b, state)
        acc = rng.integers(0, K + 1, size=N).astype(np.int32)
        gdn.gdn_decode_mtp_commit(k, a, b, e, torch.from_numpy(acc).cuda(), state)
        yh = host(y)
        for n in range(N):
            for x in ("q", "k", "v", "alpha", "beta"):
                kept[n][x].append(d[x][n, :acc[n]])
            kept[n]["y"].append(yh[n, :acc[n]])
    S_gpu = host(state)
    for n in range(N):
        cat = {x: np.concatenate(kept[n][x], axis=0)[None] for x in kept[n]}
        T = cat["q"].shape[1]
        y_ref, S_ref = gated_delta_recurrence(cat["q"], cat["k"], cat["v"], cat["alpha"], cat["beta"],
                                              S0[n:n + 1])
        say(f"  sequence {n}: {T} accepted tokens")
        if T:
            check(f"seq {n} accepted y", cat["y"], y_ref, MTP_TOL)
        check(f"seq {n} state", S_gpu[n:n + 1], S_ref, MTP_TOL)


def test_decode_workload_full_shape():
    """256 sequences x 32 heads, d = 128, bf16, 4-token drafts: every y, miss
    and committed state of two rounds; prefix states of sampled sequences."""
    say("mtp decode workload full shape")
    K = 4
    S = decode_initial_state()
    state = dev(S)
    N = S.shape[0]
    rng = np.random.default_rng(3)
    for rnd in range(2):
        d = mtp_draft_inputs(rnd, K=K)
        q, k, v, a, b = _gpu_block(d, "bf16")
        y, e, _ = gdn.gdn_decode_mtp_verify(q, k, v, a, b, state)
        acc = rng.integers(0, K + 1, size=N).astype(np.int32)
        gdn.gdn_decode_mtp_commit(k, a, b, e, torch.from_numpy(acc).cuda(), state)
        y_ref = np.empty(y.shape)
        e_ref = np.empty(e.shape)
        S_new = np.empty(S.shape)
        for n0 in range(0, N, 32):
            sl = slice(n0, n0 + 32)
            yy, ee, _ = mtp_verify(d["q"][sl], d["k"][sl], d["v"][sl], d["alpha"][sl], d["beta"][sl], S[sl])
            y_ref[sl], e_ref[sl] = yy, ee
            S_new[sl] = mtp_commit(d["k"][sl], d["alpha"][sl], d["beta"][sl], ee, acc[sl], S[sl])
        check(f"round {rnd} y", host(y), y_ref, MTP_TOL)
        check(f"round {rnd} e", host(e), e_ref, MTP_TOL)
        check(f"round {rnd} state", host(state), S_new, MTP_TOL)
        if rnd == 0:
            _, _, pref = gdn.gdn_decode_mtp_verify(q, k, v, a, b, dev(S), return_e=False,
                                                   return_prefix_states=True)
            for n in (0, 97, 255):
                _, _, p_ref = mtp_verify(d["q"][n:n + 1], d["k"][n:n + 1], d["v"][n:n + 1],
                                         d["alpha"][n:n + 1], d["beta"][n:n + 1], S[n:n + 1])
                check(f"prefix states seq {n}", host(pref[n:n + 1]), p_ref, MTP_TOL)
            del pref
        S = S_new


@pytest.mark.parametrize("K,Kp", [(4, 4), (5, 3), (1, 8)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_commit_verify_equals_commit_then_verify(K, Kp, dtype):
    """The fused call: commit the previous block's accepted prefix, then verify
    the new block, against the oracle's commit followed by its verify."""
    say(f"mtp commit+verify K={K} Kp={Kp} {dtype}")
    N, H, d_ = 6, 3, 128
    prev, S0 = _block(N, Kp, H, d_, d_, dtype, seed=40 + K)
    new, _ = _block(N, K, H, d_, d_, dtype, seed=50 + Kp)
    _, pe_ref, _ = mtp_verify(prev["q"], prev["k"], prev["v"], prev["alpha"], prev["beta"], S0)
    acc = np.array([0, Kp, 1, Kp // 2, 7, -2], dtype=np.int32)
    state = dev(S0)
    y, e = gdn.gdn_decode_mtp_commit_verify(*_gpu_block(new, dtype), state, dev(prev["k"], dtype),
                                            dev(prev["alpha"]), dev(prev["beta"]), dev(pe_ref),
                                            torch.from_numpy(acc).cuda(), scale=0.9)
    S1 = mtp_commit(prev["k"], prev["alpha"], prev["beta"], pe_ref, np.clip(acc, 0, Kp), S0)
    y_ref, e_ref, _ = mtp_verify(new["q"], new["k"], new["v"], new["alpha"], new["beta"], S1, scale=0.9)
    check("committed state", host(state), S1, MTP_TOL)
    check("y", host(y), y_ref, MTP_TOL)
    check("e", host(e), e_ref, MTP_TOL)
    np.testing.assert_array_equal(host(state)[0], S0[0].astype(np.float64))    # nothing accepted: untouched


def test_fused_rounds_follow_the_accepted_tokens():
    """Rounds of the fused call (each commits the previous round's accepted
    drafts), with a final plain commit: outputs of accepted drafts and the final
    state equal one recurrence over the accepted tokens only."""
    say("mtp fused rounds")
    N, K, H, d_ = 4, 4, 3, 64
    rng = np.random.default_rng(77)
    S0 = (0.2 * rng.standard_normal((N, H, d_, d_))).astype(np.float32)
    state = dev(S0)
    kept = [{x: [] for x in ("q", "k", "v", "alpha", "beta", "y")} for _ in range(N)]
    prev = None
    for rnd in range(5):
        d = prefill_inputs(N, K, H, d_, d_, "bf16", -1.0, 0.5, seed=[77, rnd])
        blk = _gpu_block(d, "bf16")
        if prev is None:
            y, e, _ = gdn.gdn_decode_mtp_verify(*blk, state)
        else:
            pk, pa, pb, pe, pacc = prev
            y, e = gdn.gdn_decode_mtp_commit_verify(*blk, state, pk, pa, pb, pe, pacc)
        acc = rng.integers(0, K + 1, size=N).astype(np.int32)
        prev = (blk[1], blk[3], blk[4], e, torch.from_numpy(acc).cuda())
        yh = host(y)
        for n in range(N):
            for x in ("q", "k", "v", "alpha", "beta"):
                kept[n][x].append(d[x][n, :acc[n]])
            kept[n]["y"].append(yh[n, :acc[n]])
    pk, pa, pb, pe, pacc = prev
    gdn.gdn_decode_mtp_commit(pk, pa, pb, pe, pacc, state)
    S_gpu = host(state)
    for n in range(N):
        cat = {x: np.concatenate(kept[n][x], axis=0)[None] for x in kept[n]}
        y_ref, S_ref = gated_delta_recurrence(cat["q"], cat["k"], cat["v"], cat["alpha"], cat["beta"], S0[n:n + 1])
        if cat["q"].shape[1]:
            check(f"seq {n} accepted y", cat["y"], y_ref, MTP_TOL)
        check(f"seq {n} state", S_gpu[n:n + 1], S_ref, MTP_TOL)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_commit_verify_with_e_aliasing_prev_e(dtype):
    """The fused call with e written into prev_e's own buffer (K == K_prev):
    the same state, y and e as with separate buffers."""
    say(f"mtp commit+verify, e aliasing prev_e, {dtype}")
    N, K, H, d_ = 7, 4, 3, 128
    prev, S0 = _block(N, K, H, d_, d_, dtype, seed=61)
    new, _ = _block(N, K, H, d_, d_, dtype, seed=62)
    _, pe_ref, _ = mtp_verify(prev["q"], prev["k"], prev["v"], prev["alpha"], prev["beta"], S0)
    acc = torch.from_numpy(np.array([0, K, 1, 2, 3, K, 0], dtype=np.int32)).cuda()
    pk, pa, pb = dev(prev["k"], dtype), dev(prev["alpha"]), dev(prev["beta"])
    blk = _gpu_block(new, dtype)
    state_sep = dev(S0)
    y_sep, e_sep = gdn.gdn_decode_mtp_commit_verify(*blk, state_sep, pk, pa, pb, dev(pe_ref), acc)
    state_al = dev(S0)
    shared = dev(pe_ref)
    y_al, e_al = gdn.gdn_decode_mtp_commit_verify(*blk, state_al, pk, pa, pb, shared, acc, e=shared)
    assert e_al.data_ptr() == shared.data_ptr()
    np.testing.assert_array_equal(host(state_al), host(state_sep))
    np.testing.assert_array_equal(host(y_al), host(y_sep))
    np.testing.assert_array_equal(host(e_al), host(e_sep))
    S1 = mtp_commit(prev["k"], prev["alpha"], prev["beta"], pe_ref, host(acc).astype(np.int32), S0)
    y_ref, e_ref, _ = mtp_verify(new["q"], new["k"], new["v"], new["alpha"], new["beta"], S1)
    check("aliased y", host(y_al), y_ref, MTP_TOL)
    check("aliased e", host(e_al), e_ref, MTP_TOL)
