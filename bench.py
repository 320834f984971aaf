"""Benchmark of the GDN-2 forward hot path on one MI355X.

A step is one chunkwise forward (gdn2_chunk_fwd) over the batched training
shape B=8, T=4096, H=16, dk=dv=128 (bf16 q/k/v/b/w, FP32 alpha and state,
N(0, 0.1^2) initial state).  ``value`` is its throughput in tokens/s (B*T
tokens per call), inputs resident in HBM.  The decode half of the metric --
gdn2_recurrent_step over N=256 sequences x 16 heads with 128 x 128 FP32
states, 64 consecutive in-place steps -- is timed before it and reported as
state GB/s under "decode".  The chunkwise timing starts after --settle untimed
launches (the shader clock's dip after a heavy kernel starts) and the W
warm-up ones.  Both carry their roofline; the FP64 CPU oracle is timed on a
bounded sample of the same chunkwise workload as ``cpu_baseline``.

Prints exactly one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN-2 fwd tokens/s (H16,d128,T4K,B8) + decode state GB/s; % of roofline"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak
# FP32 vector ALU without packed FP32 (which this build leaves off): 256 CUs x
# 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz
FP32_VALU_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
MFMA_FP32_PEAK_TFLOPS = 157.3  # dense FP32 matrix-core peak
NAMES = ("q", "k", "v", "alpha", "b", "w")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def chunk_bytes(B, T, H, dk, dv, N, eb=2, gates=0):
    """Algorithmic HBM bytes of one chunkwise forward: q, k, b, v, w read and
    o written in the input dtype, alpha read in FP32, the state read once and
    written once in FP32.  A scalar gate (gate layout flags 1 erase, 2 write,
    8 decay) is one value per token and head; a tied write gate (4) is not
    read."""
    tok = B * T * H
    erase = eb if gates & 1 else dk * eb
    write = 0 if gates & 4 else eb if gates & 2 else dv * eb
    gate = erase + write
    decay = 4 if gates & 8 else dk * 4
    return tok * (2 * dk * eb + dv * eb + gate + decay + dv * eb) + 2 * N * H * dk * dv * 4


def chunk_flops(lengths, H, dk, dv, C=64):
    """Triangle-aware FLOPs of the chunkwise form, summed over chunks of every
    sequence: A (strict lower) and P (lower incl. diagonal) over dk channels,
    T = (I + A)^-1 (~L^3/3), T [Et | Z], W S, Qt S, P U and Kb^T U."""
    total = 0
    for n in lengths:
        full, tail = divmod(int(n), C)
        for L, cnt in ((C, full), (tail, 1 if tail else 0)):
            per = (dk * L * (L - 1) + dk * L * (L + 1) + L ** 3 / 3 + (dk + dv) * L * (L + 1)
                   + 3 * 2 * L * dk * dv + dv * L * (L + 1))
            total += cnt * per
    return total * H


def bwd_bytes(B, T, H, dk, dv, N, eb=2):
    """Algorithmic HBM bytes of one backward call: q, k, b, v, w, d_o read and
    dq, dk, db, dv, dw written in the input dtype, alpha read and dalpha
    written in FP32, the initial state and the final-state seed read and the
    initial-state gradient written in FP32 (workspace traffic not counted)."""
    tok = B * T * H
    return tok * (6 * dk * eb + 5 * dv * eb + 2 * dk * 4) + 3 * N * H * dk * dv * 4


def bwd_flops(lengths, H, dk, dv, C=32):
    """FLOPs of the chunkwise backward at C-token chunks (32 on the FP32 path,
    64 on the matrix-core path), summed over chunks: the forward recompute
    (X, U = Tm X, the state update), the reverse pass (dU, dX, the
    state-gradient update), the key-side products (dA, dP, dEt, dQt, dKb) and
    the per-chunk algebra (A, P, Tm, pairwise)."""
    total = 0
    for n in lengths:
        full, tail = divmod(int(n), C)
        for L, cnt in ((C, full), (tail, 1 if tail else 0)):
            per = (18 * L * dk * dv + 5 * L * L * dv + 5 * L * L * dk + L ** 3 / 3 + 2 * dk * dv)
            total += cnt * per
    return total * H


def step_bytes(N, H, dk, dv, eb=2):
    """Algorithmic HBM bytes of one decode step: the FP32 state read and
    written once, the token vectors read, o written."""
    return N * H * (2 * dk * dv * 4 + 3 * dk * eb + 2 * dv * eb + dk * 4 + dv * eb)


# What the recorded HBM counters of a kernel depend on: its source file and
# the device helpers, and the argument struct it takes (comments and blank
# lines do not count).
KERNEL_SOURCES = {"chunk": ("chunk_fwd_mfma.hip", "ChunkArgs"), "decode": ("recurrent_step.hip", "StepArgs")}


def _strip_comments(text):
    import re

    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_digest(part):
    """sha256 of the code a kernel's counters depend on."""
    import hashlib
    import re

    csrc = os.path.join(ROOT, "delta_rule_linear_gdn2_amd", "csrc")
    src, struct = KERNEL_SOURCES[part]
    h = hashlib.sha256()
    for name in (src, "gdn2_device.hpp"):
        with open(os.path.join(csrc, name)) as f:
            h.update(_strip_comments(f.read()).encode())
    with open(os.path.join(csrc, "launch.hpp")) as f:
        m = re.search(r"struct %s \{.*?\};" % struct, _strip_comments(f.read()), flags=re.S)
    h.update(m.group(0).encode())
    return h.hexdigest()


def pmc_traffic(part):
    """HBM bytes per launch measured by rocprofv3 FETCH_SIZE + WRITE_SIZE
    (scaled by the copy-kernel factors) as recorded in profiles/pmc_traffic.json,
    or None when the kernel's code has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)["kernels"][part]
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes"] if rec.get("source_digest") == source_digest(part) else None


def to_dev(x, dtype):
    from delta_rule_linear_gdn2_amd import workloads as W

    return {n: W.to_torch(x[n], "f32" if n == "alpha" else dtype, "cuda") for n in NAMES}


def settle(fn, launches):
    """Untimed launches that hold the GPU under the workload's own load until
    the shader clock has settled.  The power management lowers the clock for
    a few tens of milliseconds after a heavy kernel starts (launch times rise
    by up to a fifth, then fall back), so without this the first few dozen
    launches measure the clock's transient rather than the kernel."""
    import torch

    for _ in range(launches):
        fn()
    torch.cuda.synchronize()


def time_events(fn, warmup, steps):
    """Time ``steps`` calls of fn after ``warmup`` untimed ones.

    The timed region is the ``steps`` calls back to back between one pair of
    HIP events on the current stream (bracketed by device synchronisations);
    its total (ms) and host wall time are returned.  A second, instrumented
    pass of ``steps`` calls then records an event pair around each call for
    the spread of single calls (``per``, ms each).  It is kept out of the
    timed region because each event record between launches adds a few
    microseconds of dispatch gap that is not kernel work."""
    import torch

    for _ in range(warmup):
        fn()
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record()
    for _ in range(steps):
        fn()
    t_all1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    per = [e0.elapsed_time(e1) for e0, e1 in ev]
    return per, t_all0.elapsed_time(t_all1), wall


def bench_chunk(args, pre=None):
    """Time the chunkwise forward.  ``pre`` (optional) runs after the inputs
    are on the device and before the warmup launches; its result is returned
    under "pre"."""
    import torch

    from delta_rule_linear_gdn2_amd import binding
    from delta_rule_linear_gdn2_amd import workloads as W

    t0 = time.time()
    x = W.make(args.workload)
    wl = x["workload"]
    log(f"generated {wl.name} in {time.time() - t0:.1f}s")
    d = to_dev(x, wl.dtype)
    s0 = None if x["initial_state"] is None else torch.from_numpy(x["initial_state"]).cuda()
    cu = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).cuda()
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    N = B if cu is None else int(cu.shape[0]) - 1
    o = torch.empty((B, T, H, dv), dtype=d["q"].dtype, device="cuda")
    sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device="cuda")

    def call():
        binding.gdn2_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], s0,
                               final_state=sf, out=o, cu_seqlens=cu)

    pre_res = pre() if pre is not None else None
    settle(call, getattr(args, "settle", 0))
    per, total_ms, wall = time_events(call, args.warmup, args.steps)
    ms = total_ms / args.steps  # one launch per step: also the average launch duration
    kern_ms = ms
    log("chunk per-launch us (instrumented pass): " + " ".join(f"{p * 1e3:.0f}" for p in per))
    eb = 2 if wl.dtype == "bf16" else 4
    nbytes = chunk_bytes(B, T, H, dk, dv, N, eb)
    tokens = B * T
    log(f"chunk: {ms * 1e3:.1f} us/step over {args.steps} back-to-back launches (instrumented pass: "
        f"mean {np.mean(per) * 1e3:.1f}, median {np.median(per) * 1e3:.1f}, min {min(per) * 1e3:.1f}, "
        f"max {max(per) * 1e3:.1f} us per launch), "
        f"{tokens / (ms / 1e3) / 1e6:.2f} M tokens/s, {nbytes / (kern_ms / 1e3) / 1e9:.0f} GB/s")
    return dict(x=x, wl=wl, tokens=tokens, ms=ms, kern_ms=kern_ms, wall=wall, bytes=nbytes,
                per=per, dims=(B, T, H, dk, dv, N), pre=pre_res)


def bench_decode(args, x=None):
    import torch

    from delta_rule_linear_gdn2_amd import binding
    from delta_rule_linear_gdn2_amd import workloads as W

    x = W.make("decode_b256") if x is None else x
    wl = x["workload"]
    steps_in = x["q"].shape[0]
    N, H, dk = x["q"].shape[1:]
    dv = x["v"].shape[-1]
    slices = [to_dev({n: x[n][t] for n in NAMES}, wl.dtype) for t in range(steps_in)]
    state = torch.from_numpy(x["initial_state"]).cuda()
    outs = [torch.empty((N, H, dv), dtype=slices[0]["q"].dtype, device="cuda") for _ in range(steps_in)]

    def call():  # the 64 consecutive in-place steps
        for t in range(steps_in):
            s = slices[t]
            binding.gdn2_recurrent_step(s["q"], s["k"], s["v"], s["alpha"], s["b"], s["w"], state,
                                        out=outs[t])

    per, total_ms, _ = time_events(call, max(1, args.warmup), max(1, args.steps // 4))
    step_ms = total_ms / max(1, args.steps // 4) / steps_in
    state_bytes = 2 * N * H * dk * dv * 4
    nbytes = step_bytes(N, H, dk, dv)
    log(f"decode: {step_ms * 1e3:.1f} us/step, state {state_bytes / (step_ms / 1e3) / 1e9:.0f} GB/s")
    return dict(step_ms=step_ms, state_gbps=state_bytes / (step_ms / 1e3) / 1e9,
                achieved=nbytes / (step_ms / 1e3) / 1e9, bytes=nbytes)


def bench_decode_rotated(args, nstates=4, x=None):
    """decode_b256 with ``nstates`` distinct 268 MB states in rotation: step t
    updates state t mod nstates in place, so a state was last touched
    nstates - 1 steps (and (nstates - 1) x 537 MB of other traffic) earlier and
    cannot still sit in the 256 MB Infinity Cache.  64 steps timed as one
    region, per step."""
    import torch

    from delta_rule_linear_gdn2_amd import binding
    from delta_rule_linear_gdn2_amd import workloads as W

    x = W.make("decode_b256") if x is None else x
    wl = x["workload"]
    steps_in = x["q"].shape[0]
    N, H, dk = x["q"].shape[1:]
    dv = x["v"].shape[-1]
    slices = [to_dev({n: x[n][t] for n in NAMES}, wl.dtype) for t in range(steps_in)]
    s0 = torch.from_numpy(x["initial_state"]).cuda()
    states = [s0.clone() for _ in range(nstates)]
    outs = [torch.empty((N, H, dv), dtype=slices[0]["q"].dtype, device="cuda") for _ in range(steps_in)]

    def call():
        for t in range(steps_in):
            s = slices[t]
            binding.gdn2_recurrent_step(s["q"], s["k"], s["v"], s["alpha"], s["b"], s["w"], states[t % nstates],
                                        out=outs[t])

    per, total_ms, _ = time_events(call, max(1, args.warmup), max(1, args.steps // 4))
    step_ms = total_ms / max(1, args.steps // 4) / steps_in
    state_bytes = 2 * N * H * dk * dv * 4
    nbytes = step_bytes(N, H, dk, dv)
    log(f"decode, {nstates} states in rotation: {step_ms * 1e3:.1f} us/step, "
        f"state {state_bytes / (step_ms / 1e3) / 1e9:.0f} GB/s")
    return dict(step_ms=step_ms, state_gbps=state_bytes / (step_ms / 1e3) / 1e9,
                achieved=nbytes / (step_ms / 1e3) / 1e9, bytes=nbytes,
                timing=f"{steps_in} consecutive steps over {nstates} states in rotation, per step")


def bench_decode_flushed(args, reps=20, warm=3):
    """decode_b256 one step at a time, each after a 1 GiB device write that
    evicts the state from the 256 MB Infinity Cache: the cold-cache figure
    beside the 64-step in-place headline."""
    import torch

    from delta_rule_linear_gdn2_amd import binding
    from delta_rule_linear_gdn2_amd import workloads as W

    x = W.make("decode_b256")
    wl = x["workload"]
    steps_in = x["q"].shape[0]
    N, H, dk = x["q"].shape[1:]
    dv = x["v"].shape[-1]
    slices = [to_dev({n: x[n][t] for n in NAMES}, wl.dtype) for t in range(steps_in)]
    state = torch.from_numpy(x["initial_state"]).cuda()
    out = torch.empty((N, H, dv), dtype=slices[0]["q"].dtype, device="cuda")
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for i in range(warm + reps):
        flush.fill_(float(i))
        s = slices[i % steps_in]
        e0.record()
        binding.gdn2_recurrent_step(s["q"], s["k"], s["v"], s["alpha"], s["b"], s["w"], state, out=out)
        e1.record()
        torch.cuda.synchronize()
        if i >= warm:
            times.append(e0.elapsed_time(e1))
    step_ms = float(np.median(times))
    state_bytes = 2 * N * H * dk * dv * 4
    nbytes = step_bytes(N, H, dk, dv)
    log(f"decode flushed: {step_ms * 1e3:.1f} us/step, state {state_bytes / (step_ms / 1e3) / 1e9:.0f} GB/s")
    return dict(step_ms=step_ms, state_gbps=state_bytes / (step_ms / 1e3) / 1e9,
                achieved=nbytes / (step_ms / 1e3) / 1e9, timing=f"median of {reps} single steps after {warm}")


def cpu_baseline(x, wl, chains_rows=4):
    """The FP64 oracle on the first ``chains_rows`` batch rows (all heads, full length)."""
    import oracle

    sub = {n: np.ascontiguousarray(x[n][:chains_rows]) for n in NAMES}
    s0 = None if x["initial_state"] is None else np.ascontiguousarray(x["initial_state"][:chains_rows])
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.recurrent(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["b"], sub["w"], s0, threads=threads)
    wall = time.perf_counter() - t0
    tokens = chains_rows * wl.T
    return {"value": tokens / wall, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{chains_rows} of {wl.B} sequences x all {wl.H} heads x {wl.T} tokens "
                      f"({chains_rows * wl.H} (sequence, head) chains) of the same workload, FP64, "
                      f"{wall:.1f} s wall"}


def bench_bwd(args):
    """The gate-aware backward pass on batched_bf16 (B=8, T=4096, H=16, d=128):
    median HIP-event time per call, with a final-state seed and the
    initial-state gradient."""
    import torch

    from delta_rule_linear_gdn2_amd import binding
    from delta_rule_linear_gdn2_amd import workloads as W

    x = W.make("batched_bf16")
    wl = x["workload"]
    d = to_dev(x, "bf16")
    s0 = torch.from_numpy(x["initial_state"]).cuda()
    rng = np.random.default_rng(7)
    g = W.to_torch(rng.standard_normal(x["v"].shape).astype(np.float32), "bf16", "cuda")
    gs = torch.from_numpy(rng.standard_normal(x["initial_state"].shape).astype(np.float32)).cuda()
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    ws = torch.empty(binding.gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, 0, 1), dtype=torch.uint8,
                     device="cuda")

    def call():
        binding.gdn2_chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], g, s0, gs, workspace=ws)

    per, _, _ = time_events(call, args.warmup, args.steps)
    ms = float(np.median(per))
    # 0: the bf16 matrix-core path ran; 1: a chunk was out of its range and the FP32 path ran
    path = "bf16 matrix-core" if int(ws[:4].view(torch.int32).item()) == 0 else "FP32 (range fallback)"
    nbytes = bwd_bytes(B, T, H, dk, dv, B)
    flops = bwd_flops([T] * B, H, dk, dv, C=64 if path.startswith("bf16") else 32)
    peak = MFMA_BF16_PEAK_TFLOPS if path.startswith("bf16") else MFMA_FP32_PEAK_TFLOPS
    log(f"backward ({path} path): {ms:.2f} ms per call, {B * T / (ms / 1e3) / 1e6:.2f} M tokens/s, "
        f"{flops / (ms / 1e3) / 1e12:.1f} TFLOP/s ({flops / (ms / 1e3) / 1e12 / peak * 100:.1f}% of the "
        f"{peak:.0f} TFLOP/s matrix peak), {nbytes / (ms / 1e3) / 1e9:.0f} GB/s of algorithmic bytes")
    return dict(x=x, wl=wl, ms=ms, bytes=nbytes, flops=flops, ws_bytes=ws.numel(), path=path, peak=peak)


def bench_mixer(args):
    """The token-mixer prologue (K = 4) and epilogue on batched_bf16's shape
    (B=8, T=4096, H=16, d=128, bf16): one report row each."""
    import torch

    from delta_rule_linear_gdn2_amd import binding
    from delta_rule_linear_gdn2_amd import workloads as W

    x = W.make("batched_bf16")
    B, T, H, dk, dv, K = 8, 4096, 16, 128, 128, 4
    rng = np.random.default_rng(9)
    d = to_dev(x, "bf16")
    conv = [torch.from_numpy((0.5 * rng.standard_normal((H * dd, K))).astype(np.float32)).cuda() for dd in (dk, dk, dv)]
    state = torch.zeros((B, H * (2 * dk + dv), K - 1), dtype=torch.float32, device="cuda")
    outs = {}
    rows = []

    def call_pro():
        outs["p"] = binding.gdn2_mixer_prologue(d["q"], d["k"], d["v"], conv[0], conv[1], conv[2], d["b"], d["w"],
                                                conv_state=state, q_scale=dk ** -0.5)

    per, _, _ = time_events(call_pro, args.warmup, args.steps)
    ms = float(np.median(per))
    nbytes = B * T * H * (3 * dk * 2 + 2 * dv * 2) * 2  # xq, xk, b_logit, xv, w_logit in; q, k, b, v, w out
    log(f"mixer prologue: {ms * 1e3:.1f} us, {nbytes / (ms / 1e3) / 1e9:.0f} GB/s")
    rows.append({"report": "config", "workload": "batched_bf16 token-mixer prologue (K=4)",
                 "us_per_call": ms * 1e3, "GBps": nbytes / (ms / 1e3) / 1e9,
                 "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, "algorithmic_bytes": nbytes})
    gate = d["w"]
    wgt = torch.ones(dv, dtype=torch.float32, device="cuda")
    y = torch.empty_like(d["v"])

    def call_epi():
        binding.gdn2_mixer_epilogue(d["v"], gate, wgt, out=y)

    per, _, _ = time_events(call_epi, args.warmup, args.steps)
    ms = float(np.median(per))
    nbytes = B * T * H * 3 * dv * 2  # o, gate in; y out
    log(f"mixer epilogue: {ms * 1e3:.1f} us, {nbytes / (ms / 1e3) / 1e9:.0f} GB/s")
    rows.append({"report": "config", "workload": "batched_bf16 token-mixer epilogue",
                 "us_per_call": ms * 1e3, "GBps": nbytes / (ms / 1e3) / 1e9,
                 "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, "algorithmic_bytes": nbytes})
    return rows


def run_only(args):
    """One part alone (for rocprofv3 runs); prints one JSON line."""
    import torch

    if args.only == "bwd":
        bw = bench_bwd(args)
        res = {"part": "bwd", "workload": bw["wl"].name, "median_call_ms": bw["ms"],
               "algorithmic_bytes": bw["bytes"], "flops": bw["flops"], "launches": args.steps + args.warmup}
    elif args.only == "chunk":
        ch = bench_chunk(args)
        res = {"part": "chunk", "workload": ch["wl"].name, "avg_launch_ms": ch["kern_ms"],
               "algorithmic_bytes": ch["bytes"], "launches": args.steps + args.warmup}
    elif args.only == "decode":
        dec = bench_decode(args)
        res = {"part": "decode", "us_per_step": dec["step_ms"] * 1e3, "algorithmic_bytes": dec["bytes"]}
    elif args.only == "segmented":  # layer_bf16 (16 chains) through the few-chain segmented path
        args.workload = "layer_bf16"
        ch = bench_chunk(args)
        res = {"part": "segmented", "workload": ch["wl"].name, "avg_launch_ms": ch["kern_ms"],
               "median_launch_ms": float(np.median(ch["per"])), "launches": args.steps + args.warmup}
    elif args.only == "mixer":
        res = {"part": "mixer", "rows": bench_mixer(args), "launches": args.steps + args.warmup}
    else:
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        per, total, _ = time_events(lambda: dst.copy_(src), args.warmup, args.steps)
        ms = float(np.mean(per))
        res = {"part": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "avg_launch_ms": ms,
               "GBps": 2 * nbytes / (ms / 1e3) / 1e9, "launches": args.steps + args.warmup}
    print(json.dumps(res), flush=True)


def run_configs(args):
    """Per-configuration report (not the headline line): one JSON line per
    chunkwise workload and gate mode, one for decode and one for the oracle on
    all host cores and on one.  The single-head-batch workload is timed over
    three input sets in rotation so that repeats cannot be served from the
    Infinity Cache."""
    import torch

    import oracle
    from delta_rule_linear_gdn2_amd import binding
    from delta_rule_linear_gdn2_amd import workloads as W

    full, tied, scalar = binding.GATES_FULL, binding.GATES_KDA, binding.GATES_GDN
    # (gate mode of the inputs, layout passed): the reduced-gate inputs run once
    # broadcast through the full layout and once in their compact layout
    for name, modes, rotate in (("layer_bf16", (("gdn2", full),), 3), ("long16k_bf16", (("gdn2", full),), 1),
                                ("batched_bf16", (("gdn2", full), ("kda", tied), ("gdn", scalar)), 1),
                                ("varlen32_bf16", (("gdn2", full), ("kda", full), ("kda", tied), ("gdn", full),
                                                   ("gdn", scalar)), 1)):
        for mode, gates in modes:
            sets = []
            for i in range(rotate):
                seed = None if i == 0 else W.WORKLOADS[name].seed + 100 * i
                x = W.make(name, gate_mode=mode, seed=seed)
                wl = x["workload"]
                d = to_dev(x, wl.dtype)
                d["s0"] = None if x["initial_state"] is None else torch.from_numpy(x["initial_state"]).cuda()
                d["cu"] = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).cuda()
                if gates != full:  # compact gates: beta [..], alpha [..] for scalar decay
                    d["b"] = d["b"][..., 0].contiguous()
                    d["w"] = None
                    if gates == scalar:
                        d["alpha"] = d["alpha"][..., 0].contiguous()
                    torch.cuda.synchronize()
                sets.append(d)
            B, T, H, dk = x["q"].shape
            dv = x["v"].shape[-1]
            N = B if x["cu_seqlens"] is None else len(x["cu_seqlens"]) - 1
            o = torch.empty((B, T, H, dv), dtype=sets[0]["q"].dtype, device="cuda")
            sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device="cuda")
            idx = [0]

            few = binding.gdn2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, 0 if x["cu_seqlens"] is None else N,
                                                         binding.DTYPE_BF16 if wl.dtype == "bf16" else 0) > 0

            def call(segmented=True):
                d = sets[idx[0] % rotate]
                idx[0] += 1
                binding.gdn2_chunk_fwd_gates(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], gates, d["s0"],
                                             final_state=sf, out=o, cu_seqlens=d["cu"], segmented=segmented)

            settle(call, args.settle)
            if few:  # the single pass beside the segmented path the call takes
                per1, _, _ = time_events(lambda: call(False), args.warmup, args.steps)
                single_ms = float(np.median(per1))
                log(f"{name}: single pass {single_ms * 1e3:.1f} us")
            per, _, _ = time_events(call, args.warmup, args.steps)
            kern_ms = float(np.median(per))
            nbytes = chunk_bytes(B, T, H, dk, dv, N, 2 if wl.dtype == "bf16" else 4, gates)
            if x["initial_state"] is None:  # no state to read
                nbytes -= N * H * dk * dv * 4
            layout = {full: "full", tied: "kda (flags 5)", scalar: "gdn (flags 13)"}[gates]
            row = {"report": "config", "workload": name, "gate_mode": mode, "gate_layout": layout, "tokens": B * T,
                   "sequences": N, "us_per_call": kern_ms * 1e3, "tokens_per_s": B * T / (kern_ms / 1e3),
                   "GBps": nbytes / (kern_ms / 1e3) / 1e9,
                   "hbm_frac": nbytes / (kern_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
                   "input_sets": rotate,
                   "timing": f"median of {args.steps} launches after {args.settle} settling and {args.warmup} "
                             f"warm-up launches"}
            if few:
                row["path"] = "segmented (few chains)"
                row["single_pass_us"] = single_ms * 1e3
            log(f"{name}/{mode}/{layout}: {row['us_per_call']:.1f} us, {row['tokens_per_s'] / 1e6:.1f} M tokens/s, "
                f"{row['hbm_frac'] * 100:.1f}% HBM")
            print(json.dumps(row), flush=True)
            del sets
    dec = bench_decode(args)
    print(json.dumps({"report": "config", "workload": "decode_b256", "us_per_step": dec["step_ms"] * 1e3,
                      "state_GBps": dec["state_gbps"], "hbm_frac": dec["achieved"] / HBM_PEAK_GBPS,
                      "timing": "64 consecutive in-place steps, per step"}), flush=True)
    rot = bench_decode_rotated(args)
    print(json.dumps({"report": "config", "workload": "decode_b256, four states in rotation (cache-clean)",
                      "us_per_step": rot["step_ms"] * 1e3, "state_GBps": rot["state_gbps"],
                      "hbm_frac": rot["achieved"] / HBM_PEAK_GBPS, "timing": rot["timing"]}), flush=True)
    fl = bench_decode_flushed(args)
    print(json.dumps({"report": "config", "workload": "decode_b256, Infinity Cache flushed before each step",
                      "us_per_step": fl["step_ms"] * 1e3, "state_GBps": fl["state_gbps"],
                      "hbm_frac": fl["achieved"] / HBM_PEAK_GBPS, "timing": fl["timing"]}), flush=True)
    # several tokens per sequence in one recurrent call (verification steps, short prompts)
    for T in (4, 16, 64):
        N, H, dk, dv = 256, 16, 128, 128
        x = W.make("batched_bf16", seed=2000 + T, B=N, T=T, H=H)
        d = to_dev(x, "bf16")
        state = torch.from_numpy(x["initial_state"]).cuda()  # [N, H, dk, dv], N(0, 0.1^2)
        o = torch.empty((N, T, H, dv), dtype=torch.bfloat16, device="cuda")

        def call_multi():
            binding.gdn2_recurrent_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], state, out=o)

        per, _, _ = time_events(call_multi, args.warmup, args.steps)
        kern_ms = float(np.median(per))
        nbytes = N * H * (2 * dk * dv * 4 + T * (3 * dk * 2 + 2 * dv * 2 + dk * 4 + dv * 2))
        row = {"report": "config", "workload": f"recurrent_fwd N={N} H={H} d=128 bf16 T={T}",
               "us_per_call": kern_ms * 1e3, "tokens_per_s": N * T / (kern_ms / 1e3),
               "GBps": nbytes / (kern_ms / 1e3) / 1e9, "hbm_frac": nbytes / (kern_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
               "kernel": "recurrent" if T < 24 else "chunkwise (long calls are dispatched to it)",
               "timing": f"median of {args.steps} launches after {args.warmup}"}
        log(f"recurrent_fwd T={T}: {row['us_per_call']:.1f} us, {row['tokens_per_s'] / 1e6:.2f} M tokens/s, "
            f"{row['hbm_frac'] * 100:.1f}% HBM")
        print(json.dumps(row), flush=True)
        del d, x
    # the token mixer around the recurrence on the headline shape (HBM-bound passes)
    for row in bench_mixer(args):
        print(json.dumps(row), flush=True)
    # the gate-aware backward on the headline shape, and the oracle's reverse mode beside it
    bw = bench_bwd(args)
    t0 = time.perf_counter()
    xb = bw["x"]
    sub = {n: np.ascontiguousarray(xb[n][:1, :1024, :1]) for n in NAMES}
    rng = np.random.default_rng(8)
    oracle.backward(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["b"], sub["w"],
                    rng.standard_normal(sub["v"].shape), np.ascontiguousarray(xb["initial_state"][:1, :1]),
                    rng.standard_normal((1, 1, 128, 128)), threads=1)
    one_bwd = time.perf_counter() - t0
    wlb = bw["wl"]
    print(json.dumps({"report": "config", "workload": "batched_bf16 backward (gdn2_chunk_bwd)",
                      "ms_per_call": bw["ms"], "tokens_per_s": wlb.B * wlb.T / (bw["ms"] / 1e3),
                      "GBps": bw["bytes"] / (bw["ms"] / 1e3) / 1e9,
                      "hbm_frac": bw["bytes"] / (bw["ms"] / 1e3) / 1e9 / HBM_PEAK_GBPS,
                      "path": bw["path"],
                      "TFLOPs": bw["flops"] / (bw["ms"] / 1e3) / 1e12,
                      "mfma_frac": bw["flops"] / (bw["ms"] / 1e3) / 1e12 / bw["peak"],
                      "mfma_peak_TFLOPs": bw["peak"],
                      "workspace_bytes": bw["ws_bytes"],
                      "oracle_one_core": {"value": 1024 / one_bwd, "unit": "token-heads/s",
                                          "sample": f"1 sequence x 1 head x 1024 tokens, {one_bwd:.2f} s"}}),
          flush=True)
    del bw, xb
    # the oracle: all cores on four sequences of the headline workload, one core on one (sequence, head)
    x = W.make("batched_bf16")
    wl = x["workload"]
    cpu_all = cpu_baseline(x, wl, chains_rows=4)
    sub = {n: np.ascontiguousarray(x[n][:1, :, :1]) for n in NAMES}
    s0 = np.ascontiguousarray(x["initial_state"][:1, :1])
    t0 = time.perf_counter()
    oracle.recurrent(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["b"], sub["w"], s0, threads=1)
    one = time.perf_counter() - t0
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    print(json.dumps({"report": "oracle", "cpu_model": model, "nproc": os.cpu_count(),
                      "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"),
                      "all_cores": cpu_all,
                      "one_core": {"value": wl.T / one, "unit": "token-heads/s", "cores": 1,
                                   "sample": f"1 sequence x 1 head x {wl.T} tokens, {one:.2f} s"}}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="batched_bf16",
                    choices=["batched_bf16", "layer_bf16", "long16k_bf16", "varlen32_bf16", "tiny_f32"])
    ap.add_argument("--settle", type=int, default=150,
                    help="untimed chunkwise launches before the warm-up ones, so that the timed launches run on a "
                         "settled shader clock (headline line and --configs; --only parts take none)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode half")
    ap.add_argument("--only", choices=["chunk", "decode", "copy", "bwd", "mixer", "segmented"], default=None,
                    help="profiling aid: run one part only and print its timing line "
                         "(copy = a plain 1 GiB device copy, the reference for HBM byte counters; "
                         "segmented = layer_bf16 through the few-chain segmented path)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--configs", action="store_true",
                    help="report every configuration (chunkwise workloads, gate modes, decode, oracle) "
                         "as separate JSON lines instead of the headline line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch

    from delta_rule_linear_gdn2_amd import binding

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.load()
    if args.only:
        args.settle = 0
        return run_only(args)
    if args.configs:
        return run_configs(args)
    # The decode half runs first.  The chunkwise launches that follow it still
    # ride a dip of the shader clock (the power management lowers it for a few
    # tens of milliseconds once the heavier chunkwise kernel starts), so
    # --settle untimed chunkwise launches precede the W warm-up and K timed ones.
    from delta_rule_linear_gdn2_amd import workloads as W

    xd = None if args.no_decode else W.make("decode_b256")

    def decode_first():
        if xd is None:
            return None, None
        return bench_decode(args, xd), bench_decode_rotated(args, x=xd)

    ch = bench_chunk(args, pre=decode_first)
    dec, rot = ch["pre"]
    cpu = None
    if not args.no_cpu and ch["wl"].kind == "chunk":
        cpu = cpu_baseline(ch["x"], ch["wl"], chains_rows=ch["wl"].B)
        log(f"cpu oracle: {cpu['value']:.0f} tokens/s on {cpu['cores']} threads")
    B, T, H, dk, dv, N = ch["dims"]
    wl = ch["wl"]
    achieved = ch["bytes"] / (ch["kern_ms"] / 1e3) / 1e9
    if N == B and ch["x"]["cu_seqlens"] is None:
        lengths = [T] * B
    else:
        lengths = np.diff(ch["x"]["cu_seqlens"]).tolist()
    flops = chunk_flops(lengths, H, dk, dv)
    mfma_tflops = flops / (ch["kern_ms"] / 1e3) / 1e12
    out = {
        "metric": METRIC,
        "value": ch["tokens"] / (ch["ms"] / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_launches": args.settle,
        "ms_per_step": ch["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded numpy PCG64; Gaussian/sigmoid inputs, L2-normalised q,k)",
        "config": {"workload": f"{wl.name}: chunkwise forward B={B} T={T} H={H} dk={dk} dv={dv}, "
                               f"64-token chunks, FP32 alpha/state",
                   "B": B, "T": T, "H": H, "dk": dk, "dv": dv, "num_seqs": N},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": pmc_traffic("chunk") if wl.name == "batched_bf16" else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE)",
                     "kernel": "gdn2 chunk forward", "algorithmic_bytes": ch["bytes"],
                     "avg_launch_ms": ch["kern_ms"],
                     "launch_ms": {"median": float(np.median(ch["per"])), "mean": float(np.mean(ch["per"])),
                                   "min": float(min(ch["per"])), "max": float(max(ch["per"])),
                                   "launches": len(ch["per"]),
                                   "from": "a pass of as many launches after the timed region, each "
                                           "between its own pair of HIP events"},
                     "mfma": {"achieved": mfma_tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": mfma_tflops / MFMA_BF16_PEAK_TFLOPS,
                              "flops": flops, "counting": "triangle-aware algorithmic FLOPs"}},
        "cpu_baseline": cpu,
    }
    if dec is not None:
        out["decode"] = {
            "workload": "decode_b256: N=256 H=16 dk=dv=128, bf16 tokens, FP32 state, 64 in-place steps",
            "state_GBps": dec["state_gbps"], "us_per_step": dec["step_ms"] * 1e3,
            "roofline": {"bound": "hbm", "achieved": dec["achieved"], "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": dec["achieved"] / HBM_PEAK_GBPS,
                         "traffic": pmc_traffic("decode"),
                         "traffic_unit": "HBM bytes per step (rocprofv3 FETCH_SIZE+WRITE_SIZE)",
                         "algorithmic_bytes": dec["bytes"]},
            "rotated": {"workload": "the same steps over four distinct states in rotation: each state last "
                                    "touched four steps earlier, so none is still in the 256 MB Infinity Cache",
                        "state_GBps": rot["state_gbps"], "us_per_step": rot["step_ms"] * 1e3,
                        "hbm_frac": rot["achieved"] / HBM_PEAK_GBPS},
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
