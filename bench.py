"""Benchmark of the KDA chunkwise forward on one MI355X.

A step is one kda_chunk_fwd call over the whole batch: gate (from logits),
chunk-local cumulative decay, intra-chunk products and inverse, the serial
inter-chunk state scan and the output, all inside the library's kernels. The
workload is the training-shaped batch B=8, H=32, T=8192, d_k=d_v=128, bf16,
chunk 64, zero initial state (synthetic, seeded; inputs resident in HBM).

Before the W warm-up steps, the step is run untimed for at least 200 ms
(`prewarm_ms` in the line): a fresh GPU ramps its clocks over the first
tens of launches, and a short warm-up would time that ramp. The timed loop is
unchanged by it.

Prints one JSON line. `roofline` reports the fused chunk kernel against HBM
bandwidth: algorithmic bytes per launch (q, k, v, o in bf16; gate logits and
beta in fp32; the fp32 state written once per (sequence, head)) divided by the
kernel's average duration, taken from HIP events recorded around every launch
on the stream the kernel runs on. `cpu_baseline` is the fp64 oracle timed on
the host cores on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       python bench.py --pass backward      (kda_chunk_bwd on the same workload)
       python bench.py --copy-calibration   (plain copy kernel for counter scaling)
       python bench.py --pass decode        (one decode token per (sequence, head))
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
FP32_MATRIX_PEAK_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_chunk_pipe_train8k_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "gated_delta_rule_92_amd", "csrc", f)
                  for f in ("kda_chunk_pipe.hip", "kda_common.h", "kda_internal.h")]
# the backward's three kernels: the pipelined kernel's checkpoint and reverse
# modes and the per-chunk gradient kernel
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_backward_train8k_traffic.json")
BWD_KERNEL_SOURCES = KERNEL_SOURCES + [os.path.join(ROOT, "gated_delta_rule_92_amd", "csrc",
                                                    "kda_backward.hip")]


PREWARM_MS = 200.0
PROBE_LIB = os.path.join(ROOT, "libhbm_probe.so")


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(sources=None) -> str:
    """sha256 over the kernel sources a stored counter record was taken on:
    the record is used only while the sources are unchanged."""
    h = hashlib.sha256()
    for p in (sources or KERNEL_SOURCES):
        h.update(open(p, "rb").read())
    return h.hexdigest()


def algorithmic_bytes(w, n_tokens: int, n_units: int, has_h0: bool) -> int:
    """HBM bytes the forward must move at minimum for one launch."""
    el = 2 if w.dtype_name == "bf16" else 4
    per_tok_head = (2 * w.Dk + 2 * w.Dv) * el + w.Dk * 4 + 4  # q,k | v,o | logits | beta
    state = w.Dk * w.Dv * 4 * n_units * (2 if has_h0 else 1)
    return per_tok_head * n_tokens * w.H + state


def algorithmic_flops(w, n_tokens: int) -> float:
    """Useful matrix-core flops per launch for the arrangement the bf16
    d=128 kernel runs (the state advanced every 16-token tile): per tile,
    A_kk and A_qk over d_k (2 x 2*16*16*d_k), V - (G*K)S, (G*Q)S and the
    state update over d_k x d_v (3 x 2*16*d_k*d_v), the solve and A_qk V~
    over d_v (2 x 2*16*16*d_v)."""
    P, dk, dv = 16, w.Dk, w.Dv
    per_tile = 2 * (2 * P * P * dk) + 3 * (2 * P * dk * dv) + 2 * (2 * P * P * dv)
    return per_tile / P * n_tokens * w.H


def chunk_form_flops(w, n_tokens: int) -> float:
    """Matrix-core flops of the pages' chunk form with C = 64 per token·head
    (causal 16-row tiles of the intra-chunk products, the three state
    products, the 64x64 triangular inverse): 2C(3 d_k + 2 d_v) 5/8 +
    6 d_k d_v + about 2,219 for the inverse."""
    C = w.chunk
    per = 2 * C * (3 * w.Dk + 2 * w.Dv) * 5 / 8 + 6 * w.Dk * w.Dv + 2219
    return per * n_tokens * w.H


def backward_algorithmic_bytes(w, n_tokens: int, n_units: int) -> int:
    """HBM bytes any backward must move at minimum for one call: read q, k, v,
    do (input dtype), gate logits (fp32) and beta; write dq, dk, dv (input
    dtype), dg (fp32) and dbeta; read the final-state gradient and write the
    initial-state gradient (fp32) once per (sequence, head)."""
    el = 2 if w.dtype_name == "bf16" else 4
    per_tok_head = (2 * w.Dk + 2 * w.Dv) * el + w.Dk * 4 + 4 + (2 * w.Dk + w.Dv) * el + w.Dk * 4 + 4
    return per_tok_head * n_tokens * w.H + 2 * w.Dk * w.Dv * 4 * n_units


def backward_design_bytes(w, n_tokens: int, n_units: int) -> int:
    """HBM bytes the three-kernel backward moves by design: the minimum above,
    plus the state and state-gradient checkpoints (one each per 64 tokens for
    bf16, 16 for fp32; written once, read once), U, V~ and dY (written once,
    read once), and the inputs that the two scans and the per-chunk kernel
    each read again (q, k, the gate, beta, v or dO)."""
    el = 2 if w.dtype_name == "bf16" else 4
    ct = 64 if w.dtype_name == "bf16" else 16
    ck = 2 * 2 * (n_tokens // ct) * w.H * w.Dk * w.Dv * el
    tok = 3 * 2 * n_tokens * w.H * w.Dv * el
    kin, gin, vin = w.Dk * el, w.Dk * 4 + 4, w.Dv * el     # k or q row, gate + beta, v or dO row
    scans = (kin + gin + vin) + (2 * kin + gin + vin)       # forward scan; reverse scan
    grads = 2 * kin + gin + vin                             # per-chunk kernel (q, k, gate, beta, dO)
    minimal_in = 2 * kin + gin + 2 * vin
    rereads = n_tokens * w.H * (scans + grads - minimal_in)
    return backward_algorithmic_bytes(w, n_tokens, n_units) + ck + tok + rereads


def cpu_baseline_backward(d, do, dhT, w, budget_s: float = 15.0):
    """The fp64 oracle's backward on a bounded sample of (sequence, head)
    units (each keeps T+1 states of d_k*d_v doubles, so at most 8 threads)."""
    from oracle import host_threads, oracle_backward, oracle_gate
    cores = min(host_threads(), 8)
    B, T, H = d["q"].shape[0], d["q"].shape[1], d["q"].shape[2]

    def run(units, threads):
        import torch
        sl = lambda x, n, h: x[n, :, h].cpu()  # noqa: E731
        cat = lambda name: torch.cat([sl(d[name], n, h) for (n, h) in units], 0)[None, :, None]  # noqa: E731
        q, k, v, z, b = (cat(n) for n in ("q", "k", "v", "z", "beta"))
        o = torch.cat([sl(do, n, h) for (n, h) in units], 0)[None, :, None]
        dst = torch.stack([dhT[n, h].cpu() for (n, h) in units], 0)[:, None]
        cu = torch.arange(len(units) + 1, dtype=torch.int32) * T
        g = oracle_gate(z, None, w.g_min)
        t0 = time.perf_counter()
        oracle_backward(q, k, v, g, b, o, None, dst, cu, 1.0, nthreads=threads)
        return time.perf_counter() - t0

    per_unit = run([(0, 0)], 1)
    n_units = max(cores, int(budget_s / max(per_unit, 1e-3)) // cores * cores)
    n_units = min(n_units, B * H)
    units = [(i % B, (i // B) % H) for i in range(n_units)]
    wall = run(units, cores)
    return {"value": n_units * T / wall, "unit": "tokens·heads/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{n_units} (sequence, head) units x {T} tokens of the {w.name} workload, "
                      f"fp64 token-by-token backward from stored states, {cores} threads, "
                      f"{wall:.1f} s wall"}


def cpu_baseline(d, w, budget_s: float = 25.0):
    """The fp64 oracle on a bounded sample of (sequence, head) units of the
    same workload, on the host cores this process may use (at most the host
    share of one GPU, 16 threads); returns a dict for the JSON line. The
    sample holds about `budget_s` seconds of single-thread oracle work (at most
    the whole workload). One unit is also timed on one thread: the per-core
    rate."""
    import numpy as np
    from oracle import host_threads, oracle_forward
    cores = host_threads()
    T = d["q"].shape[1]
    H = d["q"].shape[2]

    def unit_inputs(units):
        qs, ks, vs, zs, bs = [], [], [], [], []
        for (n, h) in units:
            qs.append(d["q"][n, :, h].cpu())
            ks.append(d["k"][n, :, h].cpu())
            vs.append(d["v"][n, :, h].cpu())
            zs.append(d["z"][n, :, h].cpu())
            bs.append(d["beta"][n, :, h].cpu())
        import torch
        cu = torch.tensor(np.arange(len(units) + 1) * T, dtype=torch.int32)
        cat = lambda xs: torch.cat(xs, 0)[None, :, None]  # noqa: E731
        return cat(qs), cat(ks), cat(vs), cat(zs), torch.cat(bs, 0)[None, :, None], cu

    # one unit on one thread: the per-core rate, and the size of the sample
    q, k, v, z, b, cu = unit_inputs([(0, 0)])
    t0 = time.perf_counter()
    oracle_forward(q, k, v, z, b, None, cu, None, w.g_min, 1.0, nthreads=1)
    per_unit = time.perf_counter() - t0
    n_units = max(cores, int(budget_s / max(per_unit, 1e-3)))
    n_units = max(cores, (n_units // cores) * cores)
    n_units = min(n_units, d["q"].shape[0] * H)
    units = [(i % d["q"].shape[0], (i // d["q"].shape[0]) % H) for i in range(n_units)]
    q, k, v, z, b, cu = unit_inputs(units)
    t0 = time.perf_counter()
    oracle_forward(q, k, v, z, b, None, cu, None, w.g_min, 1.0, nthreads=cores)
    wall = time.perf_counter() - t0
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"value": n_units * T / wall, "unit": "tokens·heads/s", "cores": cores,
            "kind": "oracle",
            "per_core_value": T / per_unit,
            "nproc": os.cpu_count(), "usable_cores": affinity,
            "sample": f"{n_units} (sequence, head) units x {T} tokens of the {w.name} workload, "
                      f"fp64 token-by-token recurrence, {cores} threads (host share of one GPU; "
                      f"{affinity} usable of {os.cpu_count()} cores), {wall:.1f} s wall; "
                      f"per_core_value: one unit on one thread, {per_unit:.2f} s"}


def copy_calibration(n_bytes: int = 1 << 30):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    x = torch.empty(n_bytes // 4, dtype=torch.float32, device="cuda").normal_()
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"copy calibration: {n_bytes} bytes read and {n_bytes} bytes written per copy")


def copy_bandwidth(dev, n_bytes: int = 1 << 30, reps: int = 10) -> float:
    """Rate of a plain device-to-device copy (bytes read + bytes written per
    second, GB/s): the practical ceiling next to the spec peak."""
    import torch
    x = torch.empty(n_bytes // 4, dtype=torch.float32, device=dev).normal_()
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        y.copy_(x)
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = 2 * n_bytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return gbs


def prewarm(step, min_ms: float = PREWARM_MS):
    """Runs `step` untimed until at least `min_ms` of wall time has passed
    (synchronising after each batch of launches). Returns (launches, ms)."""
    import torch
    n, t0 = 0, time.perf_counter()
    while min_ms > 0 and (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(4):
            step()
        n += 4
        torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) * 1e3


def probe_copy_bandwidth(dev, n_bytes: int = 1 << 30, reps: int = 10):
    """Rate of the hand-written HBM copy in libhbm_probe.so (bench_hbm.hip:
    four 16-byte loads in flight per lane, then the stores), best over grids
    of 256, 512 and 1024 workgroups: bytes read + bytes written per second
    (GB/s), timed with HIP events on the stream it is launched on. Returns
    (GB/s, grid) or (None, None) if the probe is not built."""
    import ctypes

    import torch
    if not os.path.exists(PROBE_LIB):
        return None, None
    lib = ctypes.CDLL(PROBE_LIB)
    lib.hbm_copy_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_int, ctypes.c_void_p]
    lib.hbm_copy_launch.restype = ctypes.c_int
    x = torch.empty(n_bytes // 4, dtype=torch.float32, device=dev).normal_()
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)
    best, best_grid = 0.0, None
    for grid in (256, 512, 1024):
        def launch():
            rc = lib.hbm_copy_launch(x.data_ptr(), y.data_ptr(), n_bytes // 16, grid,
                                     stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"hbm_copy_launch failed: {rc}")
        for _ in range(3):
            launch()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        gbs = 2 * n_bytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
        if gbs > best:
            best, best_grid = gbs, grid
    if not torch.equal(x, y):
        raise RuntimeError("hbm probe copy is wrong")
    del x, y
    torch.cuda.empty_cache()
    return best, best_grid


def _timed(step, steps, warmup, dev, prewarm_ms: float = PREWARM_MS):
    import torch
    prewarm(step, prewarm_ms)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, sorted(s.elapsed_time(e) for s, e in zip(starts, ends))


def bench_backward(args, d, w, dev):
    """One step = one kda_chunk_bwd call over the whole batch (forward scan,
    reverse scan, per-tile gradients), inputs and cotangents resident."""
    import torch
    from gated_delta_rule_92_amd import bwd_workspace_size, chunk_bwd
    B, T = d["q"].shape[0], d["q"].shape[1]
    N = d["N"]
    gen = torch.Generator(device=dev).manual_seed(2)
    do = torch.randn(d["v"].shape, generator=gen, device=dev).to(w.dtype)
    dhT = torch.randn((N, w.H, w.Dk, w.Dv), generator=gen, device=dev)
    ws = bwd_workspace_size(B, T, w.H, w.Dk, w.Dv, N, w.chunk, w.dtype)
    workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)

    def step():
        chunk_bwd(d["q"], d["k"], d["v"], d["z"], d["beta"], do, d["h0"], dhT, d["cu_seqlens"],
                  gate="logits", g_min=w.g_min, chunk=w.chunk, workspace=workspace)

    ms_per_step, launch_ms = _timed(step, args.steps, args.warmup, dev, args.prewarm_ms)
    kernel_ms = sum(launch_ms) / args.steps
    log(f"bench: backward {args.steps} steps, wall {ms_per_step:.3f} ms/step, "
        f"event {kernel_ms:.3f} ms/call")
    n_tokens = int(B * T)
    bytes_alg = backward_algorithmic_bytes(w, n_tokens, N * w.H)
    achieved = bytes_alg / (kernel_ms / 1e3) / 1e9
    traffic = None
    if os.path.exists(BWD_TRAFFIC_FILE):
        rec = json.load(open(BWD_TRAFFIC_FILE))
        if rec.get("source_sha256") == kernel_source_hash(BWD_KERNEL_SOURCES) and \
                rec.get("workload") == w.name:
            traffic = rec.get("bytes_per_call")
    cpu = None
    if not args.skip_cpu_baseline and d["cu_seqlens"] is None:
        log("bench: timing the fp64 oracle backward on a bounded sample (cpu_baseline)")
        cpu = cpu_baseline_backward(d, do, dhT, w)
    line = {
        "metric": "KDA chunk bwd tokens·heads/s (H=32,d=128,bf16,T=8K)",
        "value": n_tokens * w.H / (ms_per_step / 1e3),
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype_name,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward", "batch": int(B), "seq_len": w.T,
                   "heads": w.H, "d_k": w.Dk, "d_v": w.Dv, "chunk": w.chunk, "gate": "logits",
                   "g_min": w.g_min, "initial_state": d["h0"] is not None, "sequences": N},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "scope": "all three backward kernels of one call (HIP events around the "
                              "call); bytes = the minimum any backward must move; traffic = "
                              "FETCH_SIZE + WRITE_SIZE of the three kernels, copy-scaled",
                     "design_bytes": backward_design_bytes(w, n_tokens, N * w.H),
                     "algorithmic_bytes": bytes_alg},
        "kernel_ms": kernel_ms,
        "kernel_ms_median": launch_ms[len(launch_ms) // 2],
        "kernel_ms_min": launch_ms[0],
        "kernel_ms_max": launch_ms[-1],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_train(args, d, w, dev):
    """One step = a training step's KDA work over the whole batch: the forward
    and the backward. Timed both ways in one run: the training pair
    (kda_chunk_fwd_train, which also writes the backward's checkpoints, then
    kda_chunk_bwd_saved, which skips its first scan) and the regular pair
    (kda_chunk_fwd, then kda_chunk_bwd)."""
    import torch
    from gated_delta_rule_92_amd import (bwd_workspace_size, chunk_bwd, chunk_fwd, chunk_fwd_train,
                                         workspace_size)
    B, T = d["q"].shape[0], d["q"].shape[1]
    N = d["N"]
    gen = torch.Generator(device=dev).manual_seed(2)
    do = torch.randn(d["v"].shape, generator=gen, device=dev).to(w.dtype)
    dhT = torch.randn((N, w.H, w.Dk, w.Dv), generator=gen, device=dev)
    bws = torch.empty(max(bwd_workspace_size(B, T, w.H, w.Dk, w.Dv, N, w.chunk, w.dtype), 1),
                      dtype=torch.uint8, device=dev)
    fws = torch.empty(max(workspace_size(B, T, w.H, w.Dk, w.Dv, N, w.chunk, w.dtype), 1),
                      dtype=torch.uint8, device=dev)
    o = torch.empty(d["v"].shape, dtype=w.dtype, device=dev)
    hT = torch.empty((N, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    args_in = (d["q"], d["k"], d["v"], d["z"], d["beta"])

    def step_pair():
        chunk_fwd_train(*args_in, d["h0"], d["cu_seqlens"], gate="logits", g_min=w.g_min,
                        chunk=w.chunk, bwd_workspace=bws)
        chunk_bwd(*args_in, do, d["h0"], dhT, d["cu_seqlens"], gate="logits", g_min=w.g_min,
                  chunk=w.chunk, workspace=bws, saved=True)

    def step_regular():
        chunk_fwd(*args_in, d["h0"], d["cu_seqlens"], gate="logits", g_min=w.g_min, chunk=w.chunk,
                  o=o, final_state=hT, workspace=fws)
        chunk_bwd(*args_in, do, d["h0"], dhT, d["cu_seqlens"], gate="logits", g_min=w.g_min,
                  chunk=w.chunk, workspace=bws)

    reg_ms, reg_launch = _timed(step_regular, args.steps, args.warmup, dev, args.prewarm_ms)
    ms_per_step, launch_ms = _timed(step_pair, args.steps, args.warmup, dev, args.prewarm_ms)
    kernel_ms = sum(launch_ms) / args.steps
    reg_kernel_ms = sum(reg_launch) / args.steps
    log(f"bench: training step {args.steps} steps: kda_chunk_fwd_train + kda_chunk_bwd_saved "
        f"{kernel_ms:.3f} ms (wall {ms_per_step:.3f}); kda_chunk_fwd + kda_chunk_bwd "
        f"{reg_kernel_ms:.3f} ms (wall {reg_ms:.3f})")
    n_tokens = int(B * T)
    bytes_alg = algorithmic_bytes(w, n_tokens, N * w.H, d["h0"] is not None) + \
        backward_algorithmic_bytes(w, n_tokens, N * w.H)
    achieved = bytes_alg / (kernel_ms / 1e3) / 1e9
    line = {
        "metric": "KDA chunk fwd+bwd (training step) tokens·heads/s (H=32,d=128,bf16,T=8K)",
        "value": n_tokens * w.H / (ms_per_step / 1e3),
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype_name,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "train", "batch": int(B), "seq_len": w.T,
                   "heads": w.H, "d_k": w.Dk, "d_v": w.Dv, "chunk": w.chunk, "gate": "logits",
                   "g_min": w.g_min, "initial_state": d["h0"] is not None, "sequences": N},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "scope": "the forward and the backward of one step (HIP events around the "
                              "two calls); bytes = the forward's algorithmic bytes plus the "
                              "minimum any backward must move",
                     "algorithmic_bytes": bytes_alg},
        "kernel_ms": kernel_ms,
        "kernel_ms_median": launch_ms[len(launch_ms) // 2],
        "kernel_ms_min": launch_ms[0],
        "kernel_ms_max": launch_ms[-1],
        "regular_pair": {"kernel_ms": reg_kernel_ms, "ms_per_step": reg_ms,
                         "calls": "kda_chunk_fwd + kda_chunk_bwd"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_decode(args, d, w, dev):
    """One step = one kda_recurrent_step: a single token for every (sequence,
    head) of the workload, the fp32 state updated in place. The step reads and
    writes the whole state, so it is bound by HBM on the state bytes."""
    import torch
    from gated_delta_rule_92_amd import recurrent_step
    N = d["N"]
    if d["cu_seqlens"] is not None:
        first = d["cu_seqlens"][:-1].long()
        tok = lambda x: x[0, first].contiguous()  # noqa: E731  first token of each sequence
    else:
        tok = lambda x: x[:, 0].contiguous()  # noqa: E731
    q, k, v, z, beta = (tok(d[n]) for n in ("q", "k", "v", "z", "beta"))
    state = (d["h0"].clone() if d["h0"] is not None
             else torch.zeros((N, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev))
    o = torch.empty((N, w.H, w.Dv), dtype=w.dtype, device=dev)

    def step():
        recurrent_step(q, k, v, z, beta, state, gate="logits", g_min=w.g_min, o=o)

    ms_per_step, launch_ms = _timed(step, args.steps, args.warmup, dev, args.prewarm_ms)
    kernel_ms = sum(launch_ms) / args.steps
    el = 2 if w.dtype_name == "bf16" else 4
    units = N * w.H
    bytes_alg = units * (2 * w.Dk * w.Dv * 4 + (2 * w.Dk + 2 * w.Dv) * el + w.Dk * 4 + 4)
    achieved = bytes_alg / (kernel_ms / 1e3) / 1e9
    log(f"bench: decode {args.steps} steps, event {kernel_ms * 1e3:.1f} us/step, "
        f"{achieved:.0f} GB/s")
    cpu = None
    if not args.skip_cpu_baseline:
        # the oracle's token recurrence on one token per unit from the same
        # state, repeated for about 5 s
        from oracle import host_threads, oracle_forward
        cores = host_threads()
        hq, hk, hv, hz, hb = (x.cpu()[:, None] for x in (q, k, v, z, beta))
        h0 = state.cpu()
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 5.0:
            oracle_forward(hq, hk, hv, hz, hb, h0, None, None, w.g_min, 1.0, nthreads=cores)
            reps += 1
        wall = time.perf_counter() - t0
        cpu = {"value": units * reps / wall, "unit": "tokens·heads/s", "cores": cores,
               "kind": "oracle",
               "sample": f"{reps} decode steps of all {units} (sequence, head) units of the "
                         f"{w.name} workload, fp64 token recurrence, {cores} threads, "
                         f"{wall:.1f} s wall"}
    line = {
        "metric": "KDA decode step tokens·heads/s (H=32,d=128,bf16)",
        "value": units / (ms_per_step / 1e3),
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype_name,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "decode", "sequences": N, "heads": w.H,
                   "d_k": w.Dk, "d_v": w.Dv, "gate": "logits", "g_min": w.g_min},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "scope": "one kda_recurrent_step launch; bytes = state read and written "
                              "once plus the token's inputs and output"},
        "kernel_ms": kernel_ms,
        "kernel_ms_median": launch_ms[len(launch_ms) // 2],
        "kernel_ms_min": launch_ms[0],
        "kernel_ms_max": launch_ms[-1],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_gate(args, d, w, dev):
    """One step = one kda_gate launch over the whole workload: the gate
    g = g_min * sigmoid(z) and its chunk-local inclusive cumsum, fp32 in and
    out (4 + 4 bytes per element)."""
    from gated_delta_rule_92_amd import gate
    z = d["z"]
    out = torch_empty_like(z)

    def step():
        gate(z, None, w.g_min, w.chunk, d["cu_seqlens"], out=out)

    ms_per_step, launch_ms = _timed(step, args.steps, args.warmup, dev, args.prewarm_ms)
    kernel_ms = sum(launch_ms) / args.steps
    elems = z.numel()
    bytes_alg = 8 * elems
    achieved = bytes_alg / (kernel_ms / 1e3) / 1e9
    log(f"bench: gate {args.steps} steps, event {kernel_ms:.3f} ms/launch, {achieved:.0f} GB/s")
    cpu = None
    if not args.skip_cpu_baseline:
        # the oracle's gate and chunk cumsum on a bounded sample: the first
        # 4096 tokens of the first sequence, repeated for about 3 s
        from oracle import oracle_cumsum, oracle_gate
        rows = min(int(z.shape[1]), 4096)
        zs = z[:1, :rows].cpu()
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 3.0:
            oracle_cumsum(oracle_gate(zs, None, w.g_min), w.chunk)
            reps += 1
        wall = time.perf_counter() - t0
        cpu = {"value": reps * rows * w.H / wall, "unit": "tokens·heads/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{reps} passes over {rows} tokens x {w.H} heads x {w.Dk} channels of "
                         f"the {w.name} workload, fp64 gate then chunk cumsum, one thread, "
                         f"{wall:.1f} s wall"}
    n_tokens = int(z.shape[0] * z.shape[1])
    line = {
        "metric": "KDA gate + chunk cumsum tokens·heads/s (H=32,d=128)",
        "value": n_tokens * w.H / (ms_per_step / 1e3),
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "gate", "heads": w.H, "d_k": w.Dk,
                   "chunk": w.chunk, "g_min": w.g_min},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "scope": "one kda_gate launch; bytes = z read and g written once (fp32)"},
        "kernel_ms": kernel_ms,
        "kernel_ms_median": launch_ms[len(launch_ms) // 2],
        "kernel_ms_min": launch_ms[0],
        "kernel_ms_max": launch_ms[-1],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def torch_empty_like(x):
    import torch
    return torch.empty_like(x)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--workload", default="train8k")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--prewarm-ms", type=float, default=PREWARM_MS,
                    help="untimed launches before the warm-up steps, in ms of wall time (0: none; "
                         "counter runs under a profiler use 0)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--gate", choices=["logits", "softplus"], default="logits",
                    help="logits: g = g_min sigmoid(z), diagonal tiles on matrix cores; softplus: "
                         "the earlier unbounded gate -softplus(z), diagonal tiles by position pairs")
    ap.add_argument("--epilogue", choices=["none", "fused", "separate"], default="none",
                    help="add the output epilogue sigmoid(gate) * RMSNorm(o): fused into the "
                         "chunk kernel, or as a second kernel after it")
    ap.add_argument("--split", type=int, default=1,
                    help="cut every sequence into this many segments that run in parallel "
                         "(state maps + composition + re-run); 1 = the plain forward")
    ap.add_argument("--pass", dest="which",
                    choices=["forward", "backward", "train", "decode", "gate"], default="forward",
                    help="forward: kda_chunk_fwd (the default line); backward: kda_chunk_bwd with "
                         "seeded normal output and final-state gradients; train: forward and "
                         "backward of a training step, kda_chunk_fwd_train + kda_chunk_bwd_saved "
                         "next to kda_chunk_fwd + kda_chunk_bwd; decode: one "
                         "kda_recurrent_step for every (sequence, head); gate: one kda_gate "
                         "(gate and chunk-local cumsum) over the workload's logits")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path is built); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    if args.copy_calibration:
        copy_calibration()
        return 0

    from gated_delta_rule_92_amd import (chunk_fwd, chunk_fwd_gated, chunk_fwd_split, gated_rmsnorm,
                                         workspace_size)
    from gated_delta_rule_92_amd.inputs import make_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: generating workload {args.workload} on {torch.cuda.get_device_name(dev)}")
    d = make_workload(args.workload, device=dev)
    w = d["workload"]
    n_tokens = int(d["q"].shape[0] * d["q"].shape[1])
    N = d["N"]
    ws = workspace_size(d["q"].shape[0], d["q"].shape[1], w.H, w.Dk, w.Dv, N, w.chunk, w.dtype)
    workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    o = torch.empty(d["v"].shape, dtype=w.dtype, device=dev)
    hT = torch.empty((N, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)

    if args.which == "backward":
        return bench_backward(args, d, w, dev)
    if args.which == "train":
        return bench_train(args, d, w, dev)
    if args.which == "decode":
        return bench_decode(args, d, w, dev)
    if args.which == "gate":
        return bench_gate(args, d, w, dev)

    if args.epilogue != "none":
        gen = torch.Generator(device=dev).manual_seed(1)
        out_gate = torch.randn(d["v"].shape, generator=gen, device=dev).to(w.dtype)
        norm_w = torch.ones(w.Dv, device=dev)
        y = torch.empty_like(o)

    def step():
        if args.epilogue == "fused":
            chunk_fwd_gated(d["q"], d["k"], d["v"], d["z"], d["beta"], out_gate, norm_w, 1e-6,
                            d["h0"], d["cu_seqlens"], gate="logits", g_min=w.g_min, chunk=w.chunk,
                            y=y, final_state=hT, workspace=workspace)
            return
        if args.split > 1:
            chunk_fwd_split(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], d["cu_seqlens"],
                            segments=args.split, gate="logits", g_min=w.g_min, chunk=w.chunk)
            return
        chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["beta"], d["h0"], d["cu_seqlens"],
                  gate=args.gate, g_min=w.g_min, chunk=w.chunk, o=o, final_state=hT,
                  workspace=workspace)
        if args.epilogue == "separate":
            gated_rmsnorm(o, out_gate, norm_w, 1e-6, y=y)

    prewarm_n, prewarm_ms = prewarm(step, args.prewarm_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    launch_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    kernel_ms = sum(launch_ms) / args.steps
    log(f"bench: {args.steps} steps, wall {ms_per_step:.3f} ms/step, event {kernel_ms:.3f} ms/launch")

    # pieces of the context split kda_chunk_fwd took by itself for long dense
    # sequences (its workspace then opens with the piece table: the starts of
    # the first sequence's pieces, the first piece ending at T closing it)
    segments, piece_tokens = args.split, None
    if args.split == 1 and args.epilogue == "none" and d["cu_seqlens"] is None and ws >= 4 * 66:
        table = workspace[:4 * 66].view(torch.int32).cpu().tolist()
        if table[0] == 0 and 0 < table[1] <= w.T and w.T in table[1:]:
            segments = table[1:].index(w.T) + 1
            if segments > 1:
                # first, second and last piece (the first-out schedule's first
                # piece is longer, the last takes the rest)
                piece_tokens = [table[1], table[2] - table[1], w.T - table[segments - 1]]
    tok_heads = n_tokens * w.H
    value = tok_heads / (ms_per_step / 1e3)
    bytes_alg = algorithmic_bytes(w, n_tokens, N * w.H, d["h0"] is not None)
    achieved = bytes_alg / (kernel_ms / 1e3) / 1e9
    flops = algorithmic_flops(w, n_tokens)
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("source_sha256") == kernel_source_hash() and rec.get("workload") == w.name:
            traffic = rec.get("bytes_per_launch")

    torch_copy_gbs = copy_bandwidth(dev)
    probe_gbs, probe_grid = probe_copy_bandwidth(dev)
    copy_gbs = probe_gbs if probe_gbs else torch_copy_gbs
    log(f"bench: hand-written copy {probe_gbs or 0:.0f} GB/s (grid {probe_grid}), torch copy "
        f"{torch_copy_gbs:.0f} GB/s; kernel at {achieved / copy_gbs:.1%} of the first")

    cpu = None
    if not args.skip_cpu_baseline and d["cu_seqlens"] is None:
        log("bench: timing the fp64 oracle on a bounded sample (cpu_baseline)")
        cpu = cpu_baseline(d, w)

    peak_tf = BF16_DENSE_PEAK_TFLOPS if w.dtype_name == "bf16" else FP32_MATRIX_PEAK_TFLOPS
    line = {
        "metric": "KDA chunk fwd tokens·heads/s (H=32,d=128,bf16,T=8K); % MFMA peak",
        "value": value,
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype_name,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": int(d["q"].shape[0]), "seq_len": w.T, "heads": w.H,
                   "d_k": w.Dk, "d_v": w.Dv, "chunk": w.chunk, "gate": args.gate,
                   "g_min": w.g_min, "initial_state": d["h0"] is not None,
                   "sequences": N, "segments": segments, "epilogue": args.epilogue,
                   **({"piece_tokens": piece_tokens} if piece_tokens else {})},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "mfma_peak_frac": chunk_form_flops(w, n_tokens) / (kernel_ms / 1e3) / (peak_tf * 1e12),
        "mfma_peak_frac_tile_form": flops / (kernel_ms / 1e3) / (peak_tf * 1e12),
        "copy_gbs": copy_gbs,
        "copy_kind": "hand-written copy (bench_hbm.hip), best grid" if probe_gbs else "torch copy",
        "torch_copy_gbs": torch_copy_gbs,
        "frac_of_copy": achieved / copy_gbs,
        "prewarm_ms": prewarm_ms,
        "prewarm_launches": prewarm_n,
        "kernel_ms": kernel_ms,
        "kernel_ms_median": launch_ms[len(launch_ms) // 2],
        "kernel_ms_min": launch_ms[0],
        "kernel_ms_max": launch_ms[-1],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
