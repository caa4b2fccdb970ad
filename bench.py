"""Throughput of the GDN token-mixer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the hot path over the long-prefill workload
(B=1, H=32, T=32768, d_k=d_v=128, bf16 q/k/v, fp32 alpha/beta/state): the
chunked prefill kernel (gdn_prefill_fwd) followed by the gated RMSNorm
epilogue (gdn_gated_rmsnorm) on its output.  ``value`` is prefill tokens/s of
the whole step.  The same run measures the decode step on the decode workload
(256 sequences x 32 heads, d = 128, fp32 states, 1000 consecutive steps) as
state GB/s, and times the float64 CPU oracle on a bounded sample of the
prefill workload.  Rank 0 prints one JSON line.
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s at T=32K + decode state GB/s, as % of MI355X roofline"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
FP32_MFMA_PEAK_TFLOPS = 157.3


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_bytes(B, T, H, dk, dv, in_bytes=2, with_final_state=True, with_initial_state=False):
    """Algorithmic HBM bytes of one prefill call: q, k, v read once, alpha and
    beta read once, y (fp32) written once, states read/written once."""
    per_token_head = (2 * dk + dv) * in_bytes + 8 + 4 * dv
    state = 4 * dk * dv * B * H
    return B * T * H * per_token_head + state * (int(with_final_state) + int(with_initial_state))


def prefill_flops(B, T, H, dk, dv, C=64):
    """Dense MFMA tile work per token-head of the chunked form as the kernels
    evaluate it (a chunk of C tokens: K K^T, Q K^T, the (C x C)(C x d_v)
    products T' R and P E, and the three state products K S, Q S and K^T E;
    the diagonal-block inverse is left out): 6 d^2 + 8 C d at d_k = d_v = d.
    The misses E = T'(V - diag(gamma) K S) take one C x C product where the
    unfolded WY form, W = T diag(beta gamma) K and U = T diag(beta) V followed
    by U - W S, takes two, hence prefill_flops_unfolded's 6 d^2 + 10 C d."""
    return B * T * H * (2 * 2 * C * dk + 2 * 2 * C * dv + 3 * 2 * dk * dv)


def prefill_flops_unfolded(B, T, H, dk, dv, C=64):
    """The same count with separate W and U products (one more C x C x d_k)."""
    return prefill_flops(B, T, H, dk, dv, C) + B * T * H * 2 * 2 * C * dk


def bwd_bytes(B, T, H, dk, dv, in_bytes=2):
    """Algorithmic HBM bytes of one backward call: q, k, v, alpha, beta and dy
    read once, dq, dk, dv (fp32), dalpha and dbeta written once."""
    return B * T * H * ((2 * dk + dv) * in_bytes + 8 + 4 * dv + 4 * (2 * dk + dv) + 8)


def bwd_flops(B, T, H, d, C=64):
    """MFMA tile work of the four backward passes per token-head (fp16 operands
    for bf16 inputs, fp32 for fp32 inputs): the
    C x d x d products (K S, K^T E, K dS', Q^T dY, K^T dR and the three X1..X3
    contractions over d_v) and the C x C x d ones (the two Gram products, T R,
    P^T dY, T^T dE, X4, X5 and the four C x C by C x d products of dq, dk)."""
    return B * T * H * 2 * (8 * d * d + 11 * C * d)


def norm_bytes(rows, dv, in_bytes=2):
    return rows * dv * (4 + 2 * in_bytes)


PREFILL_SOURCES = ("linear_attention_recurrence_rule_amd/csrc/prefill_chunked.hip",
                   "linear_attention_recurrence_rule_amd/csrc/gdn_device.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_long_T32K_traffic.md")


def prefill_source_hash():
    h = hashlib.sha256()
    for rel in PREFILL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per prefill call from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's readings), or None when
    there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            fields = dict(line.split(":", 1) for line in f if line.startswith(("traffic_bytes_per_call:",
                                                                             "source_hash:")))
    except OSError:
        return None
    if fields.get("source_hash", "").strip() != prefill_source_hash():
        return None
    return float(fields["traffic_bytes_per_call"])


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


_POOL_DATA = {}


def _oracle_heads(h0, h1):
    """Worker of the pooled CPU baseline: the oracle over heads h0 .. h1-1 of
    the sample in _POOL_DATA (inherited through fork), one thread."""
    from threadpoolctl import threadpool_limits
    from oracle import gated_delta_recurrence
    d = _POOL_DATA
    sl = (slice(None), slice(None), slice(h0, h1))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        gated_delta_recurrence(d["q"][sl], d["k"][sl], d["v"][sl], d["alpha"][sl], d["beta"][sl])
        return time.perf_counter() - t0


def cpu_oracle_baseline(sample, H, Ts, max_workers=16):
    """Time the float64 oracle on `sample` (B=1, Ts tokens, H heads): once on
    one core, then as a process pool over heads on the cores this process may
    use (at most max_workers).  Returns the cpu_baseline object."""
    import concurrent.futures
    import multiprocessing
    from threadpoolctl import threadpool_limits
    from oracle import gated_delta_recurrence
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        gated_delta_recurrence(sample["q"], sample["k"], sample["v"], sample["alpha"], sample["beta"])
        t_one = time.perf_counter() - t0
    cores = max(1, min(max_workers, len(os.sched_getaffinity(0)), H))
    _POOL_DATA.clear()
    _POOL_DATA.update(sample)
    bounds = [(H * i // cores, H * (i + 1) // cores) for i in range(cores)]
    ctx = multiprocessing.get_context("fork")
    t0 = time.perf_counter()
    with concurrent.futures.ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as ex:
        list(ex.map(_oracle_heads, *zip(*bounds)))
    t_pool = time.perf_counter() - t0
    _POOL_DATA.clear()
    model = cpu_model()
    return {"value": Ts / t_pool, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "single_core_value": Ts / t_one,
            "sample": f"float64 numpy oracle over the first {Ts} tokens of the long-prefill workload shape "
                      f"(B=1, H={H}, d=128): {t_one:.1f} s on 1 core; {t_pool:.1f} s as a pool of {cores} "
                      f"processes over heads (pool start-up included); CPU: {model}"}


def calibrate_copy(nbytes=1 << 30, reps=4):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}), flush=True)


def _time_calls(fn, reps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_prefill_short(dev, stream, to_dev, reps=20):
    """B=4, H=16, T=4096 prefill (one call, zero initial state, final state out)."""
    import torch
    import linear_attention_recurrence_rule_amd as gdn
    from workloads import CONFIGS, config_prefill_inputs
    c = CONFIGS[1]
    B, T, H, dk, dv = c["B"], c["T"], c["H"], c["dk"], c["dv"]
    log(f"prefill short: B={B} T={T} H={H}")
    d = config_prefill_inputs(1)
    q, k, v = (to_dev(d[n], True) for n in ("q", "k", "v"))
    alpha, beta = to_dev(d["alpha"], False), to_dev(d["beta"], False)
    y = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(B, T, H, dk, dv, torch.bfloat16), dtype=torch.uint8,
                     device=dev)
    ms = _time_calls(lambda: gdn.gdn_prefill_fwd(q, k, v, alpha, beta, None, S, y, workspace=ws, stream=stream),
                     reps, 3, stream)
    nb = prefill_bytes(B, T, H, dk, dv)
    gbps = nb / (ms * 1e-3) / 1e9
    log(f"prefill short {ms * 1e3:.1f} us, {gbps:.0f} GB/s")
    return {"workload": f"GDN prefill, B={B} T={T} H={H} d={dk}, bf16 q/k/v, fp32 state and y",
            "avg_call_ms": ms, "tokens_per_s": B * T / (ms * 1e-3), "algorithmic_bytes_per_call": nb,
            "achieved": gbps, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
            "mfma_frac_of_bf16_peak": prefill_flops(B, T, H, dk, dv) / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}


def bench_prefill_segmented(dev, stream, to_dev, reps=3, distinct=8):
    """B=1, H=16, T=262144 as 64 calls of 4096 tokens carrying the state through
    initial_state/final_state (in place).  The first `distinct` 4096-token
    segments of the workload are resident and cycled over the 64 calls."""
    import torch
    import linear_attention_recurrence_rule_amd as gdn
    from workloads import CONFIGS, config_prefill_inputs
    c = CONFIGS[4]
    T, H, dk, dv, seg = c["T"], c["H"], c["dk"], c["dv"], c["segment"]
    nseg = T // seg
    log(f"prefill 262K: H={H}, {nseg} segments of {seg}")
    segs = []
    for s in range(distinct):
        d = config_prefill_inputs(4, T=seg, t_begin=s * seg)
        segs.append(tuple(to_dev(d[n], True) for n in ("q", "k", "v"))
                    + (to_dev(d["alpha"], False), to_dev(d["beta"], False)))
    y = torch.empty((1, seg, H, dv), dtype=torch.float32, device=dev)
    S = torch.zeros((1, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(1, seg, H, dk, dv, torch.bfloat16), dtype=torch.uint8,
                     device=dev)

    def sequence():
        for i in range(nseg):
            q, k, v, a, b = segs[i % distinct]
            gdn.gdn_prefill_fwd(q, k, v, a, b, S, S, y, workspace=ws, stream=stream)
    ms = _time_calls(sequence, reps, 1, stream)
    nb = nseg * prefill_bytes(1, seg, H, dk, dv, with_initial_state=True)
    gbps = nb / (ms * 1e-3) / 1e9
    log(f"prefill 262K segmented {ms:.3f} ms, {gbps:.0f} GB/s")
    return {"workload": f"GDN prefill, one {T}-token sequence, H={H} d={dk}, as {nseg} calls of {seg} tokens "
                        "carrying the state", "avg_sequence_ms": ms, "avg_call_ms": ms / nseg,
            "tokens_per_s": T / (ms * 1e-3), "algorithmic_bytes": nb, "achieved": gbps, "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "mfma_frac_of_bf16_peak": prefill_flops(1, T, H, dk, dv) / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-frontend", action="store_true")
    ap.add_argument("--no-mtp", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-qsa", action="store_true")
    ap.add_argument("--no-other-prefill", action="store_true",
                    help="skip the 4K-token and 262K-token segmented prefill workloads")
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the hot path is per "
              "(sequence, head): sequences or heads split across GPUs with no communication inside the "
              "mixer, so one GPU's share runs exactly the kernels measured here.",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return

    from workloads import (CONFIGS, config_prefill_inputs, decode_initial_state, decode_step_inputs,
                           mtp_draft_inputs)

    # ---------------- float64 CPU oracle on a bounded sample ----------------
    # (first, before anything touches the GPU, so that the worker processes are
    # forked from a process without a GPU context)
    cpu_baseline = None
    if not args.no_cpu_baseline:
        Ts, Hs = args.cpu_tokens, CONFIGS[2]["H"]
        log(f"cpu oracle: B=1 H={Hs} T={Ts} (one core, then a pool over heads)")
        ds = config_prefill_inputs(2, T=Ts)
        cpu_baseline = cpu_oracle_baseline(ds, Hs, Ts)
        del ds
        log(f"cpu oracle {cpu_baseline['single_core_value']:.1f} tokens/s on one core, "
            f"{cpu_baseline['value']:.1f} tokens/s on {cpu_baseline['cores']} cores")

    import torch
    import linear_attention_recurrence_rule_amd as gdn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gdn.load_library()

    # ---------------- prefill + epilogue (the timed step) ----------------
    c = CONFIGS[2]
    B, T, H, dk, dv = c["B"], c["T"], c["H"], c["dk"], c["dv"]
    log(f"generating prefill inputs B={B} T={T} H={H} d={dk}")
    d = config_prefill_inputs(2)

    def to_dev(x, bf16):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        return t.to(torch.bfloat16) if bf16 else t

    q, k, v, z = (to_dev(d[n], True) for n in ("q", "k", "v", "z"))
    alpha, beta = to_dev(d["alpha"], False), to_dev(d["beta"], False)
    del d
    y = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    out = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    ev = []

    def step(record):
        if record:
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record(stream)
        gdn.gdn_prefill_fwd(q, k, v, alpha, beta, None, S, y, stream=stream)
        if record:
            e1.record(stream)
        gdn.gdn_gated_rmsnorm(y, z, None, 1e-6, out, stream=stream)
        if record:
            e2.record(stream)
            ev.append((e0, e1, e2))

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    prefill_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    norm_ms = float(np.mean([b.elapsed_time(c_) for _, b, c_ in ev]))
    tokens = B * T
    value = tokens / (ms_step * 1e-3)
    pf_bytes = prefill_bytes(B, T, H, dk, dv)
    pf_gbps = pf_bytes / (prefill_ms * 1e-3) / 1e9
    pf_tflops = prefill_flops(B, T, H, dk, dv) / (prefill_ms * 1e-3) / 1e12
    pf_tflops_unf = prefill_flops_unfolded(B, T, H, dk, dv) / (prefill_ms * 1e-3) / 1e12
    nb = norm_bytes(B * T * H, dv)
    log(f"step {ms_step:.3f} ms; prefill kernel {prefill_ms:.3f} ms ({pf_gbps:.0f} GB/s); "
        f"epilogue {norm_ms:.3f} ms")

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "GDN prefill, long sequence, + gated RMSNorm epilogue",
                   "B": B, "T": T, "H": H, "d_k": dk, "d_v": dv, "chunk": 64,
                   "qkv_dtype": "bf16", "state_dtype": "fp32", "y_dtype": "fp32",
                   "epilogue_out_dtype": "bf16"},
        "roofline": {"bound": "hbm", "kernel": "gdn_prefill_fwd (prep_kernel + main_kernel)",
                     "achieved": pf_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": pf_gbps / HBM_PEAK_GBPS, "traffic": measured_traffic(),
                     "algorithmic_bytes_per_launch": pf_bytes, "avg_launch_ms": prefill_ms,
                     "mfma_tflops": pf_tflops, "mfma_frac_of_bf16_peak": pf_tflops / BF16_MFMA_PEAK_TFLOPS,
                     "mfma_frac_of_bf16_peak_unfolded_count": pf_tflops_unf / BF16_MFMA_PEAK_TFLOPS},
        "epilogue": {"kernel": "gated_rmsnorm_kernel", "avg_launch_ms": norm_ms,
                     "achieved": nb / (norm_ms * 1e-3) / 1e9, "unit": "GB/s",
                     "frac": nb / (norm_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS},
    }
    del q, k, v, z, alpha, beta, y, out
    torch.cuda.empty_cache()

    # ---------------- the 4K and 262K workloads ----------------
    if not args.no_other_prefill:
        result["prefill_short"] = bench_prefill_short(dev, stream, to_dev)
        result["prefill_262k_segmented"] = bench_prefill_segmented(dev, stream, to_dev)
        torch.cuda.empty_cache()

    # ---------------- decode: state GB/s over consecutive steps ----------------
    if not args.no_decode:
        c3 = CONFIGS[3]
        N, H3, d3 = c3["N"], c3["H"], c3["dk"]
        log(f"decode: N={N} H={H3} d={d3}, {args.decode_steps} steps")
        state = to_dev(decode_initial_state(), False)
        n_inputs = 8   # distinct seeded step inputs, cycled
        steps_in = []
        for s in range(n_inputs):
            di = decode_step_inputs(s)
            steps_in.append(tuple(to_dev(di[n], True) for n in ("q", "k", "v"))
                            + (to_dev(di["alpha"], False), to_dev(di["beta"], False)))
        yd = torch.empty((N, H3, d3), dtype=torch.float32, device=dev)
        for s in range(5):
            gdn.gdn_decode_step(*steps_in[s % n_inputs], state, yd, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.decode_steps):
            gdn.gdn_decode_step(*steps_in[s % n_inputs], state, yd, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        step_ms = e0.elapsed_time(e1) / args.decode_steps
        state_bytes = 2 * N * H3 * d3 * d3 * 4
        all_bytes = state_bytes + N * H3 * (3 * d3 * 2 + 8 + 4 * d3)
        gbps = state_bytes / (step_ms * 1e-3) / 1e9
        log(f"decode step {step_ms * 1e3:.1f} us, state {gbps:.0f} GB/s")
        result["decode"] = {"workload": "decode, 256 sequences x 32 heads, d=128, fp32 state",
                            "steps": args.decode_steps, "us_per_step": step_ms * 1e3,
                            "state_GBps": gbps, "peak": HBM_PEAK_GBPS, "frac": gbps / HBM_PEAK_GBPS,
                            "all_bytes_GBps": all_bytes / (step_ms * 1e-3) / 1e9,
                            "tokens_per_s": N / (step_ms * 1e-3)}
        del state, steps_in, yd
        torch.cuda.empty_cache()

    # ---------------- backward of the prefill on the same workload ----------------
    if not args.no_bwd:
        log(f"backward: B={B} T={T} H={H} d={dk}")
        d = config_prefill_inputs(2)
        q, k, v = (to_dev(d[n], True) for n in ("q", "k", "v"))
        alpha, beta = to_dev(d["alpha"], False), to_dev(d["beta"], False)
        del d
        gen = torch.Generator(device=dev)
        gen.manual_seed(11)
        dy = torch.randn((B, T, H, dv), generator=gen, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        outs = (torch.empty((B, T, H, dk), **f32), torch.empty((B, T, H, dk), **f32),
                torch.empty((B, T, H, dv), **f32), torch.empty((B, T, H), **f32), torch.empty((B, T, H), **f32),
                torch.empty((B, H, dk, dv), **f32))
        ws = torch.empty(gdn.gdn_prefill_bwd_workspace_bytes(B, T, H, dk, dv, torch.bfloat16), dtype=torch.uint8,
                         device=dev)

        def bwd_call():
            gdn.gdn_prefill_bwd(q, k, v, alpha, beta, dy, workspace=ws, out=outs, stream=stream)
        for _ in range(2):
            bwd_call()
        torch.cuda.synchronize()
        n_b = 5
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_b):
            bwd_call()
        e1.record(stream)
        torch.cuda.synchronize()
        b_ms = e0.elapsed_time(e1) / n_b
        bb, bf = bwd_bytes(B, T, H, dk, dv), bwd_flops(B, T, H, dk)
        result["backward"] = {"workload": f"backward of the long prefill, B={B} T={T} H={H} d={dk}, bf16 inputs, "
                                          "fp32 gradients",
                              "kernels": "bwd_prep; prep_kernel + main_kernel in its state-saving mode (chunk-start "
                                         "states); rev_walk_kernel (state gradients); bwd_grads",
                              "avg_call_ms": b_ms, "tokens_per_s": B * T / (b_ms * 1e-3),
                              "algorithmic_bytes": bb, "GBps": bb / (b_ms * 1e-3) / 1e9,
                              "hbm_frac": bb / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                              "mfma_operands": "fp16 (bf16 inputs), fp32 accumulation",
                              "mfma_tflops": bf / (b_ms * 1e-3) / 1e12,
                              "mfma_frac_of_fp16_peak": bf / (b_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}
        log(f"backward {b_ms:.3f} ms ({bf / (b_ms * 1e-3) / 1e12:.1f} TFLOP/s fp16 MFMA, "
            f"{bb / (b_ms * 1e-3) / 1e9:.0f} GB/s algorithmic)")
        del q, k, v, alpha, beta, dy, outs, ws
        torch.cuda.empty_cache()

    # ---------------- multi-token decode: verify a 4-token draft block, commit ----------------
    if not args.no_mtp:
        c3 = CONFIGS[3]
        N, H3, d3, K = c3["N"], c3["H"], c3["dk"], 4
        log(f"multi-token decode: N={N} H={H3} d={d3}, {K}-token drafts")
        state = to_dev(decode_initial_state(), False)
        blocks = []
        for r in range(4):
            di = mtp_draft_inputs(r, K=K)
            blocks.append(tuple(to_dev(di[n], True) for n in ("q", "k", "v"))
                          + (to_dev(di["alpha"], False), to_dev(di["beta"], False)))
        ym = torch.empty((N, K, H3, d3), dtype=torch.float32, device=dev)
        em = torch.empty_like(ym)
        all_acc = torch.full((N,), K, dtype=torch.int32, device=dev)
        n_rounds = 200

        def timed(fn):
            for r in range(3):
                fn(r)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for r in range(n_rounds):
                fn(r)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n_rounds

        def verify(r):
            q_, k_, v_, a_, b_ = blocks[r % len(blocks)]
            gdn.gdn_decode_mtp_verify(q_, k_, v_, a_, b_, state, y=ym, e=em, stream=stream)

        def commit(r):
            q_, k_, v_, a_, b_ = blocks[r % len(blocks)]
            gdn.gdn_decode_mtp_commit(k_, a_, b_, em, all_acc, state, stream=stream)

        def round_(r):
            verify(r)
            commit(r)

        e_prev = torch.zeros_like(em)

        def fused(r):
            # commit block r - 1 (all accepted) and verify block r in one pass
            q_, k_, v_, a_, b_ = blocks[r % len(blocks)]
            _, pk_, _, pa_, pb_ = blocks[(r - 1) % len(blocks)]
            gdn.gdn_decode_mtp_commit_verify(q_, k_, v_, a_, b_, state, pk_, pa_, pb_, e_prev, all_acc, y=ym,
                                             e=e_prev, stream=stream)
        v_ms, c_ms, r_ms, f_ms = timed(verify), timed(commit), timed(round_), timed(fused)
        sb = N * H3 * d3 * d3 * 4
        tok_io = N * H3 * K * (3 * d3 * 2 + 8)
        v_bytes = sb + tok_io + 2 * N * H3 * K * d3 * 4                  # state, q/k/v/gates, y and e
        c_bytes = 2 * sb + N * H3 * K * (d3 * 2 + 8 + d3 * 4)              # state in/out, k, gates, e
        result["mtp"] = {"workload": f"multi-token decode, {N} sequences x {H3} heads, d={d3}, {K}-token drafts, "
                                     "all accepted", "verify_us": v_ms * 1e3, "commit_us": c_ms * 1e3,
                         "round_us": r_ms * 1e3, "fused_round_us": f_ms * 1e3,
                         "fused_round_GBps": (2 * sb + tok_io + 2 * N * H3 * K * d3 * 4) / (f_ms * 1e-3) / 1e9,
                         "verify_GBps": v_bytes / (v_ms * 1e-3) / 1e9,
                         "verify_frac": v_bytes / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "commit_GBps": c_bytes / (c_ms * 1e-3) / 1e9,
                         "commit_frac": c_bytes / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "tokens_per_s": N * K / (f_ms * 1e-3)}
        log(f"mtp verify {v_ms * 1e3:.1f} us ({v_bytes / (v_ms * 1e-3) / 1e9:.0f} GB/s), "
            f"commit {c_ms * 1e3:.1f} us ({c_bytes / (c_ms * 1e-3) / 1e9:.0f} GB/s), round {r_ms * 1e3:.1f} us, "
            f"fused round {f_ms * 1e3:.1f} us")
        del state, blocks, ym, em
        torch.cuda.empty_cache()

    # ---------------- front end: projected streams -> q, k, v, alpha, beta ----------------
    if not args.no_frontend:
        W = 4
        log(f"front end: B={B} T={T} H={H} d={dk} conv width {W}")
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        fe = dict(q_proj=torch.randn((B, T, H, dk), generator=gen, device=dev).to(torch.bfloat16),
                  k_proj=torch.randn((B, T, H, dk), generator=gen, device=dev).to(torch.bfloat16),
                  v_proj=torch.randn((B, T, H, dv), generator=gen, device=dev).to(torch.bfloat16),
                  conv_q=torch.randn((H, dk, W), generator=gen, device=dev) / 2,
                  conv_k=torch.randn((H, dk, W), generator=gen, device=dev) / 2,
                  conv_v=torch.randn((H, dv, W), generator=gen, device=dev) / 2,
                  a_logit=torch.randn((B, T, H), generator=gen, device=dev),
                  b_logit=torch.randn((B, T, H), generator=gen, device=dev),
                  A=torch.full((H,), -2.0, device=dev), b_alpha=torch.full((H,), 0.5, device=dev))
        outs = (torch.empty((B, T, H, dk), dtype=torch.bfloat16, device=dev),
                torch.empty((B, T, H, dk), dtype=torch.bfloat16, device=dev),
                torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev),
                torch.empty((B, T, H), device=dev), torch.empty((B, T, H), device=dev))

        def fe_call():
            gdn.gdn_frontend_fwd(fe["q_proj"], fe["k_proj"], fe["v_proj"], fe["conv_q"], fe["conv_k"],
                                 fe["conv_v"], fe["a_logit"], fe["b_logit"], fe["A"], fe["b_alpha"],
                                 out=outs, stream=stream)
        for _ in range(3):
            fe_call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_fe = 20
        e0.record(stream)
        for _ in range(n_fe):
            fe_call()
        e1.record(stream)
        torch.cuda.synchronize()
        fe_ms = e0.elapsed_time(e1) / n_fe
        fe_bytes = B * T * H * ((2 * dk + dv) * 2 * 2 + 4 * 4)
        result["frontend"] = {"workload": f"front end, B={B} T={T} H={H} d={dk}, conv width {W}, bf16",
                              "kernel": "frontend qkv_kernel (q, k and v passes in one launch)", "avg_call_ms": fe_ms,
                              "algorithmic_bytes_per_call": fe_bytes,
                              "achieved": fe_bytes / (fe_ms * 1e-3) / 1e9, "unit": "GB/s",
                              "frac": fe_bytes / (fe_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                              "tokens_per_s": B * T / (fe_ms * 1e-3)}
        log(f"front end {fe_ms * 1e3:.1f} us, {fe_bytes / (fe_ms * 1e-3) / 1e9:.0f} GB/s")
        del fe, outs
        torch.cuda.empty_cache()

    # ---------------- QSA indexer: 64K tokens, 4 query heads, r = 4, K = 2048 ----------------
    if not args.no_qsa:
        nq, Hq, Dq, rq, Kq = 65536, 4, 128, 4, 2048
        log(f"qsa indexer: n={nq} H={Hq} D={Dq} r={rq} K={Kq}")
        gen = torch.Generator(device=dev)
        gen.manual_seed(13)
        qp = torch.randn((1, nq, Hq, Dq), generator=gen, device=dev).to(torch.bfloat16)
        kp = torch.randn((1, nq, Dq), generator=gen, device=dev).to(torch.bfloat16)
        qo = torch.empty_like(qp)
        ko = torch.empty((1, nq // rq, Dq), dtype=torch.bfloat16, device=dev)
        KBq = -(-Kq // rq)
        idx = torch.empty((1, nq, KBq), dtype=torch.int32, device=dev)
        wsq = torch.empty(gdn.gdn_qsa_select_workspace_bytes(1, nq, Hq, Dq, rq, Kq, torch.bfloat16),
                          dtype=torch.uint8, device=dev)

        def prep():
            gdn.gdn_qsa_prep(qp, kp, r=rq, out=(qo, ko), stream=stream)

        def select():
            gdn.gdn_qsa_select(qo, ko, r=rq, K=Kq, block_idx=idx, workspace=wsq, stream=stream)

        def time_it(fn, reps=10):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps
        p_ms, s_ms = time_it(prep), time_it(select)
        cand = sum((i + 1) // rq for i in range(nq))          # scored (query, block) pairs
        flops = cand * Hq * Dq * 2
        prep_bytes = (nq * Hq * Dq + nq * Dq) * 2 + (nq * Hq * Dq + (nq // rq) * Dq) * 2
        result["qsa"] = {"workload": f"QSA indexer, n={nq} tokens, {Hq} query heads, D={Dq}, r={rq}, K={Kq}, bf16",
                         "prep_ms": p_ms, "prep_GBps": prep_bytes / (p_ms * 1e-3) / 1e9,
                         "select_ms": s_ms, "scored_pairs": cand,
                         "score_tflops_over_select": flops / (s_ms * 1e-3) / 1e12,
                         "queries_per_s": nq / ((p_ms + s_ms) * 1e-3)}
        log(f"qsa prep {p_ms * 1e3:.1f} us, select {s_ms:.3f} ms ({flops / (s_ms * 1e-3) / 1e12:.1f} TFLOP/s "
            f"of score work over the whole select)")
        del qp, kp, qo, ko, idx, wsq
        torch.cuda.empty_cache()

    if cpu_baseline is not None:
        result["cpu_baseline"] = cpu_baseline

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
