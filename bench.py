#!/usr/bin/env python3
"""Benchmark of the FP8 delayed-scaling linear-layer path on one MI355X.

One step = one training iteration of an FP8 linear layer at the GPT-175B QKV projection shape
of one TP=2 rank (tokens M = 8192 = seq 2048 x batch 4, K = 12288, N = 18432), every kernel
of the path in the order a training iteration runs them:
  forward : cast+transpose x (E4M3), cast+transpose W (E4M3), FP8 GEMM + bias -> y (bf16)
  backward: dbias + cast+transpose dy (E5M2), dgrad GEMM -> dx (bf16), wgrad GEMM -> dW (fp32)
  recipe  : fused amax-history scale update of the three tensors (history length 1024)
Inputs are seeded synthetic bf16 tensors already resident in HBM; the step time includes
every launch.  `value` is the three GEMMs' 2*M*N*K FLOPs per step over the step time.

Also reported (own timings, HIP events on the launch stream):
  * per-kernel average durations inside the timed steps, the GEMM roofline fraction;
  * cast+transpose sweep at [1024, 1024], [4096, 4096] and [8192, 12288] with cold caches
    (GB/s, % of 8 TB/s), and warm back-to-back for reference at the two larger shapes;
  * dbias+cast+transpose of dy [8192, 4096] and the T=3, L=1024 scale update;
  * the forward-only small layer ([128,256] x [256,256]): eager and graph-replay latency;
  * N-chunked GEMM+bias M=8192, K=N=12288 in 4 and 8 chunks on their own streams, as a graph;
  * the lazy transpose-cache fill of FP8 codes at the weight [18432, 12288] and activation
    [8192, 12288] shapes, cold (GB/s);
  * the FP8-output GEMM (E5M2 output, own scale, amax capture) at the dgrad shape, against the
    bfloat16-output GEMM on the same operands;
  * a plain 1 GiB device copy, cold: the box's own streaming ceiling for the cast kernels;
  * the CPU oracle, one thread and threaded over row blocks on the host cores (baseline only):
    the cast family at full size (small layer, cast+transpose sweep, backward prep) and a
    bounded sample of the step.
"Cold" cast timings rotate over enough buffer sets that every launch reads input and writes
output last touched more than 1 GiB of traffic earlier (beyond the 256 MB Infinity Cache and
the L2s), with back-to-back launches between one pair of events, so the average is the
kernel's own duration (comparable with a profiler's kernel trace).
`--casts-only` runs only the cast-family timings (for an isolated profiler trace).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
FP8_PEAK = 5.0e15          # FLOP/s, MI355X dense FP8 MFMA

M, K, N = 8192, 12288, 18432
HIST_L = 1024
CT_SHAPES = [(1024, 1024), (4096, 4096), (8192, 12288)]   # cast+transpose sweep
PREP_SHAPE = (8192, 4096)                                 # backward prep: dy


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-extras", action="store_true", help="only the timed training step")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--traffic-probe", action="store_true",
                   help="only launch one plain 1 GiB device copy and one forward GEMM (for rocprofv3 --pmc "
                        "FETCH_SIZE / WRITE_SIZE passes: the copy calibrates the counters)")
    p.add_argument("--small-only", action="store_true",
                   help="only the small-layer forward [128,256] x [256,256] (for a kernel trace)")
    p.add_argument("--casts-only", action="store_true",
                   help="only the cold cast-family timings (cast+transpose sweep, cast+amax, backward prep), "
                        "printed as one JSON line (for an isolated rocprofv3 kernel trace)")
    return p.parse_args()


def traffic_probe():
    """One plain copy of 1 GiB (known traffic: 1 GiB read + 1 GiB written), one forward GEMM
    launch at the QKV shape, one cast+transpose of x [8192,12288] and one dbias+cast+transpose of
    dy [8192,4096], nothing else on the GPU, so per-dispatch counters can be compared.  Last, a
    GEMM whose operand reads are known: A [16384, 12288] against B [256, 12288], 64 tiles of one
    tile column, so each A byte is read by one workgroup only (201.3 MB) and B (3.1 MB) by at
    most the 8 L2s: the GEMM's direct-to-LDS buffer loads must read between 204.5 and 226.5 MB
    below the L2, which checks the counter scaling the copy calibrates for this access type."""
    import torch

    import fp8_delayed_scaling_amd as F

    F.lib()
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(11)
    src = torch.randint(0, 256, (1 << 30,), dtype=torch.uint8, generator=g).to(dev)
    dst = torch.empty_like(src)
    a8 = (torch.randint(0, 256, (M, K), dtype=torch.uint8, generator=g) & 0xF7).to(dev)
    b8 = (torch.randint(0, 256, (N, K), dtype=torch.uint8, generator=g) & 0xF7).to(dev)
    bias = torch.zeros(N, device=dev, dtype=torch.bfloat16)
    y = torch.empty((M, N), device=dev, dtype=torch.bfloat16)
    one = torch.ones(1, device=dev)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    F.fp8_gemm_bias(a8, F.E4M3, one, b8, F.E4M3, one, bias, y)
    torch.cuda.synchronize()
    del a8, b8, y
    # inputs drawn on the device: no further copy dispatches beside the calibration copy
    gd = torch.Generator(device=dev).manual_seed(12)
    x = torch.randn((M, K), device=dev, generator=gd).to(torch.bfloat16)
    x8, x8t = torch.empty((M, K), dtype=torch.uint8, device=dev), torch.empty((K, M), dtype=torch.uint8, device=dev)
    sinv, am = torch.zeros(1, device=dev), torch.zeros(1, device=dev)
    torch.cuda.synchronize()
    F.fp8_cast_transpose(x, torch.full((1,), 0.4, device=dev), F.E4M3, x8, x8t, sinv, am)
    torch.cuda.synchronize()
    del x, x8, x8t
    R, C = 8192, 4096
    dy = (torch.randn((R, C), device=dev, generator=gd) * 0.01).to(torch.bfloat16)
    d8, d8t = torch.empty((R, C), dtype=torch.uint8, device=dev), torch.empty((C, R), dtype=torch.uint8, device=dev)
    db = torch.empty(C, device=dev)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(R, C), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    F.fp8_dbias_cast_transpose(dy, torch.full((1,), 4096.0, device=dev), F.E5M2, d8, d8t, db, ws, sinv, am)
    torch.cuda.synchronize()
    del dy, d8, d8t, db, ws
    Mc, Nc = 16384, 256
    a8 = (torch.randint(0, 256, (Mc, K), dtype=torch.uint8, device=dev, generator=gd) & 0xF7)
    b8 = (torch.randint(0, 256, (Nc, K), dtype=torch.uint8, device=dev, generator=gd) & 0xF7)
    yc = torch.empty((Mc, Nc), device=dev, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    F.fp8_gemm_bias(a8, F.E4M3, one, b8, F.E4M3, one, None, yc)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_probe": "done", "copy_bytes_each_way": 1 << 30, "gemm": [M, N, K],
                      "cast_transpose": [M, K], "dbias_cast_transpose": [R, C],
                      "calibration_gemm": [Mc, Nc, K]}))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.traffic_probe:
        traffic_probe()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; sharding across GPUs is described, "
                                   "not implemented (run with --gpus 1)"}))
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_delayed_scaling_amd as F
    import synthetic as S

    F.lib()   # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.small_only:
        print(json.dumps({"small_only": {"small_forward_128x256x256": small_forward(F, S, torch, np, dev, bf16)}}))
        return

    if args.casts_only:
        res = cast_family(F, S, torch, np, dev, bf16)
        res["roofline_cast_transpose"] = _cast_roofline(res["cast_transpose_sweep_cold"]["8192x12288"])
        print(json.dumps({"casts_only": res}))
        return

    t0 = time.time()
    x_h = S.normal_bf16(S.seed_for(4, 0), (M, K), 1.0)
    w_h = S.normal_bf16(S.seed_for(4, 1), (N, K), 0.02)
    b_h = S.normal_bf16(S.seed_for(4, 2), (N,), 0.1)
    dy_h = S.normal_bf16(S.seed_for(4, 3), (M, N), 0.01)
    x, w, b, dy = bf16(x_h), bf16(w_h), bf16(b_h), bf16(dy_h)
    log(f"inputs generated and uploaded in {time.time() - t0:.1f}s")

    u8 = dict(device=dev, dtype=torch.uint8)
    f32 = dict(device=dev, dtype=torch.float32)
    hist = torch.zeros((HIST_L, 3), **f32)
    scale = torch.ones(3, **f32)
    scale_inv = torch.ones(3, **f32)
    sinv = torch.zeros(3, **f32)
    x8, x8t = torch.empty((M, K), **u8), torch.empty((K, M), **u8)
    w8, w8t = torch.empty((N, K), **u8), torch.empty((K, N), **u8)
    dy8, dy8t = torch.empty((M, N), **u8), torch.empty((N, M), **u8)
    y = torch.empty((M, N), device=dev, dtype=torch.bfloat16)
    dx = torch.empty((M, K), device=dev, dtype=torch.bfloat16)
    dw = torch.empty((N, K), **f32)
    db = torch.empty(N, **f32)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(M, N), **u8)
    fmts = [F.E4M3, F.E4M3, F.E5M2]

    names = ["cast_transpose_x", "cast_transpose_w", "gemm_fwd", "dbias_cast_transpose_dy", "gemm_dgrad",
             "gemm_wgrad", "scale_update"]

    def step(ev=None):
        """One training iteration; `ev` (list of event pairs) brackets each launch when given."""
        calls = [
            lambda: F.fp8_cast_transpose(x, scale[0:1], F.E4M3, x8, x8t, sinv[0:1], hist[0, 0:1]),
            lambda: F.fp8_cast_transpose(w, scale[1:2], F.E4M3, w8, w8t, sinv[1:2], hist[0, 1:2]),
            lambda: F.fp8_gemm_bias(x8, F.E4M3, sinv[0:1], w8, F.E4M3, sinv[1:2], b, y),
            lambda: F.fp8_dbias_cast_transpose(dy, scale[2:3], F.E5M2, dy8, dy8t, db, ws, sinv[2:3], hist[0, 2:3]),
            lambda: F.fp8_gemm_bias(dy8, F.E5M2, sinv[2:3], w8t, F.E4M3, sinv[1:2], None, dx),
            lambda: F.fp8_gemm_bias(dy8t, F.E5M2, sinv[2:3], x8t, F.E4M3, sinv[0:1], None, dw),
            lambda: F.fp8_scale_update(hist, scale, scale_inv, fmts, 0),
        ]
        for i, c in enumerate(calls):
            if ev is not None:
                ev[i][0].record()
            c()
            if ev is not None:
                ev[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K steps, events around every launch
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
           for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for s in range(args.steps):
        step(evs[s])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    per_kernel = {n: float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]))
                  for i, n in enumerate(names)}
    gemm_flop = 2.0 * M * N * K
    step_flop = 3 * gemm_flop
    value = step_flop / (ms_step * 1e-3) / 1e12
    gemm_ms = float(np.mean([per_kernel["gemm_fwd"], per_kernel["gemm_dgrad"], per_kernel["gemm_wgrad"]]))
    gemm_tflops = gemm_flop / (gemm_ms * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms ({value:.1f} TFLOP/s), per kernel ms: "
        + ", ".join(f"{k}={v:.4f}" for k, v in per_kernel.items()))

    # the same step captured once into a hipGraph (every launch of the step, no host sync, no
    # memset nodes) and replayed K times
    cap = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        step()
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(args.steps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / args.steps
    del graph

    # bytes of the cast kernels (algorithmic: read bf16, write two FP8 copies)
    ct_x_bytes = M * K * 4
    ct_w_bytes = N * K * 4
    dct_bytes = M * N * 4 + N * 4

    traffic = _traffic_record("gemm_fp8_qkv_counters.json", "gemm.hip")

    result = {
        "metric": "FP8 linear fwd+bwd TFLOP/s + cast_transpose GB/s, % of MI355X peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded normal bf16: x~N(0,1), W~N(0,0.02), bias~N(0,0.1), dy~N(0,0.01))",
        "config": {
            "workload": "FP8 linear training step, GPT-175B QKV projection at one TP=2 rank's share: "
                        "M=8192 tokens (seq 2048 x batch 4), K=12288, N=18432; fwd + bwd + scale update",
            "M": M, "K": K, "N": N, "amax_history": HIST_L, "formats": "x,W E4M3; dy E5M2",
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "k_gemm_pipe16 (fwd/dgrad/wgrad average)",
            "achieved": round(gemm_tflops, 2),
            "peak": FP8_PEAK / 1e12,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops * 1e12 / FP8_PEAK, 4),
            "traffic": traffic,
        },
        "kernels_ms": {k: round(v, 4) for k, v in per_kernel.items()},
        "step_breakdown": {
            "gemm_tflops_each": {k: round(gemm_flop / (per_kernel[k] * 1e-3) / 1e12, 1)
                                 for k in ("gemm_fwd", "gemm_dgrad", "gemm_wgrad")},
            "cast_transpose_x_GBps": round(ct_x_bytes / (per_kernel["cast_transpose_x"] * 1e-3) / 1e9, 1),
            "cast_transpose_w_GBps": round(ct_w_bytes / (per_kernel["cast_transpose_w"] * 1e-3) / 1e9, 1),
            "dbias_cast_transpose_dy_GBps": round(dct_bytes / (per_kernel["dbias_cast_transpose_dy"] * 1e-3) / 1e9, 1),
            "gemm_only_tflops": round(step_flop / (3 * gemm_ms * 1e-3) / 1e12, 1),
            "host_wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
            "graph_replay_ms_per_step": round(graph_ms, 4),
            "graph_replay_tflops": round(step_flop / (graph_ms * 1e-3) / 1e12, 1),
        },
    }
    del evs

    if not args.no_extras:
        result["extras"] = extras(F, S, torch, np, dev, bf16,
                                  {"x8": x8, "w8": w8, "w8t": w8t, "dy8": dy8, "sinv": sinv})
        result["roofline_cast_transpose"] = _cast_roofline(result["extras"]["cast_transpose_sweep_cold"]["8192x12288"])

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(x_h, w_h, b_h, dy_h)

    print(json.dumps(result))


def _traffic_record(counters, source):
    """HBM traffic per launch from a committed rocprofv3 counter summary under profiles/, if it
    was taken on the current kernel source (its sha256 is stored with the counters); else null."""
    path = os.path.join(ROOT, "profiles", counters)
    src = os.path.join(ROOT, "fp8_delayed_scaling_amd", "csrc", source)
    try:
        rec = json.load(open(path))
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if rec.get("source_sha256", rec.get("gemm_source_sha256")) != h:
            return None
        return rec.get("traffic_bytes_per_launch")
    except (OSError, ValueError):
        return None


def _cast_roofline(cold):
    """Roofline entry of the cast+transpose of x [8192, 12288] (cold): 4 algorithmic bytes per
    element (2 read, 1 + 1 written) over the kernel's average duration, against 8 TB/s."""
    gbps = cold["GBps"]
    return {"bound": "hbm", "kernel": "k_cast_transpose (x [8192,12288] E4M3, cold)", "achieved": gbps,
            "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(gbps * 1e9 / HBM_PEAK, 4),
            "traffic": _traffic_record("cast_transpose_counters.json", "cast.hip")}


def _time_fn(torch, fn, reps=20):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


ROTATE_BYTES = 1 << 30     # traffic between two touches of one buffer set in the cold timings


def cold_rotating(torch, calls, bytes_per_call, reps=5):
    """Average duration (ms) of one call when its buffers are cold: `calls` are the same
    operation on distinct buffer sets, launched round-robin back to back, so a set is touched
    again only after the others' traffic (at least ROTATE_BYTES in total) has passed through
    the caches.  One warm-up pass over the sets, then `reps` passes between one pair of events."""
    for c in calls:
        c()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        for c in calls:
            c()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / (reps * len(calls))


def _abi(F, torch, name, *args):
    """One call of a C-ABI entry point with its arguments marshalled once (tensors as device
    addresses, the current stream last): what a C caller pays per call, without the Python
    binding's checks, so short kernels are timed rather than the host."""
    fn = getattr(F.lib(), name)
    raw = [a.data_ptr() if isinstance(a, torch.Tensor) else a for a in args]
    raw.append(torch.cuda.current_stream().cuda_stream)

    def call():
        st = fn(*raw)
        if st != 0:
            raise RuntimeError(f"{name}: {F.fp8ds_status_string(st)}")
    return call


def _nsets(bytes_per_call):
    """Buffer sets for cold_rotating: the others' traffic exceeds ROTATE_BYTES, at least 3 sets."""
    return max(3, 1 + -(-ROTATE_BYTES // bytes_per_call))


def cast_family(F, S, torch, np, dev, bf16):
    """Cold timings of the cast family at the sweep and backward-prep workloads: cast+transpose
    of N(0,1) tensors with 0.1% outliers x1e3 at [1024,1024], [4096,4096], [8192,12288] (at the
    steady-state scale 0.4); cast+amax at [8192,12288]; dbias+cast+transpose of dy [8192,4096]
    ~N(0,0.01) (E5M2, scale 4096) and the T=3, L=1024 scale update.  Every call goes through the
    C ABI with its arguments marshalled once (`_abi`)."""
    out = {}
    u8 = dict(device=dev, dtype=torch.uint8)
    f32 = dict(device=dev, dtype=torch.float32)
    sweep = {}
    for idx, (R, C) in enumerate([(1024, 1024), (4096, 4096), (8192, 12288)]):
        xd = bf16(S.outlier_bf16(S.seed_for(1, idx), (R, C), 1.0))
        nbytes = R * C * 4
        ns = _nsets(nbytes)
        # distinct inputs per set: copies of the one seeded tensor (same bytes, other addresses)
        xs = [xd] + [xd.clone() for _ in range(ns - 1)]
        sets = [(x_, torch.empty((R, C), **u8), torch.empty((C, R), **u8)) for x_ in xs]
        sc, si, am = torch.tensor([0.4], **f32), torch.zeros(1, **f32), torch.zeros(1, **f32)
        calls = [_abi(F, torch, "fp8_cast_transpose", x_, R, C, sc, F.E4M3, o, ot, si, am, None) for x_, o, ot in sets]
        ms = cold_rotating(torch, calls, nbytes)
        gbps = nbytes / (ms * 1e-3) / 1e9
        sweep[f"{R}x{C}"] = {"us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                             "frac_hbm": round(gbps * 1e9 / HBM_PEAK, 3), "buffer_sets": ns}
        if R * C >= 4096 * 4096:
            # warm, for reference: back-to-back calls on one set, the input partly cache-resident
            msw = _time_fn(torch, calls[0], 20)
            sweep[f"{R}x{C}"].update({"warm_us": round(msw * 1e3, 2), "warm_GBps": round(nbytes / (msw * 1e-3) / 1e9, 1)})
        del xs, sets, calls, xd
    out["cast_transpose_sweep_cold"] = sweep

    # cast+amax (row-major only) at the large shape, cold
    R, C = 8192, 12288
    xd = bf16(S.outlier_bf16(S.seed_for(1, 2), (R, C), 1.0))
    nbytes = R * C * 3
    xs = [xd] + [xd.clone() for _ in range(_nsets(nbytes) - 1)]
    sets = [(x_, torch.empty((R * C,), **u8)) for x_ in xs]
    sc, si, am = torch.tensor([0.4], **f32), torch.zeros(1, **f32), torch.zeros(1, **f32)
    ms = cold_rotating(torch, [_abi(F, torch, "fp8_cast_amax", x_, R * C, sc, F.E4M3, o, si, am, None) for x_, o in sets],
                       nbytes)
    out["cast_amax_8192x12288_cold"] = {"us": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                        "frac_hbm": round(nbytes / (ms * 1e-3) / HBM_PEAK, 3)}
    del xs, sets, xd

    # backward prep: dbias + cast+transpose dy [8192, 4096] E5M2, cold; scale update L=1024, T=3
    R, C = 8192, 4096
    dyd = bf16(S.normal_bf16(S.seed_for(3, 0), (R, C), 0.01))
    nbytes = R * C * 4 + C * 4
    xs = [dyd] + [dyd.clone() for _ in range(_nsets(nbytes) - 1)]
    sets = [(x_, torch.empty((R, C), **u8), torch.empty((C, R), **u8), torch.empty(C, **f32),
             torch.zeros(F.fp8_dbias_workspace_bytes(R, C), **u8)) for x_ in xs]
    sc, si, am = torch.tensor([4096.0], **f32), torch.zeros(1, **f32), torch.zeros(1, **f32)
    ms = cold_rotating(torch, [_abi(F, torch, "fp8_dbias_cast_transpose", x_, R, C, sc, F.E5M2, o, ot, si, am, d, w,
                                    w.numel()) for x_, o, ot, d, w in sets], nbytes)
    h = torch.from_numpy(S.log_uniform_f32(S.seed_for(3, 1), 1024 * 3, 1e-3, 1e3).reshape(1024, 3)).to(dev)
    s3, si3 = torch.ones(3, **f32), torch.ones(3, **f32)
    F.fp8_scale_update(h, s3, si3, [0, 0, 1], 0)
    torch.cuda.synchronize()
    fmts = (ctypes.c_int32 * 3)(0, 0, 1)
    us_upd = _time_fn(torch, _abi(F, torch, "fp8_scale_update", h, 1024, 3, s3, si3, ctypes.cast(fmts, ctypes.c_void_p), 0),
                      50) * 1e3
    out["backward_prep"] = {"dbias_cast_transpose_8192x4096_us": round(ms * 1e3, 2),
                            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                            "frac_hbm": round(nbytes / (ms * 1e-3) / HBM_PEAK, 3),
                            "scale_update_L1024_T3_us": round(us_upd, 2)}
    del xs, sets, dyd
    torch.cuda.empty_cache()
    return out


def small_forward(F, S, torch, np, dev, bf16):
    """The small layer [128,256] x [256,256] (bias, E4M3, one launch): host time per call back to
    back through the binding, a prepared call, the C ABI with its arguments marshalled once, a
    torch graph replay and hipGraphLaunch of the same graph."""
    f32 = dict(device=dev, dtype=torch.float32)
    u8 = dict(device=dev, dtype=torch.uint8)
    Ms, Ns, Ks = 128, 256, 256
    xs, wsm, bs = bf16(S.normal_bf16(S.seed_for(0, 0), (Ms, Ks), 1.0)), bf16(S.normal_bf16(S.seed_for(0, 1), (Ns, Ks), 1.0)), \
        bf16(S.normal_bf16(S.seed_for(0, 2), (Ns,), 0.1))
    hs, ss, sis = torch.zeros((16, 3), **f32), torch.ones(3, **f32), torch.zeros(3, **f32)
    x8s, w8s, w8ts = torch.empty((Ms, Ks), **u8), torch.empty((Ns, Ks), **u8), torch.empty((Ks, Ns), **u8)
    ys = torch.empty((Ms, Ns), device=dev, dtype=torch.bfloat16)

    def small_fwd(stream=None):
        F.fp8_linear_fwd(xs, wsm, bs, ss[0:1], hs[0, 0:1], x8s, None, sis[0:1], ss[1:2], hs[0, 1:2], w8s, w8ts,
                         sis[1:2], None, ys, stream=stream)

    small_fwd()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(200):
        small_fwd()
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t) / 200 * 1e6
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        small_fwd(stream=cap)
    g.replay()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(200):
        g.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t) / 200 * 1e6
    # the same call through the C ABI directly with its arguments marshalled once (what a C
    # caller pays per call; the difference is the Python binding's argument checks)
    L = F.lib()
    raw_args = [xs.data_ptr(), wsm.data_ptr(), bs.data_ptr(), Ms, Ns, Ks, ss[0:1].data_ptr(), hs[0, 0:1].data_ptr(),
                x8s.data_ptr(), None, sis[0:1].data_ptr(), ss[1:2].data_ptr(), hs[0, 1:2].data_ptr(), w8s.data_ptr(),
                w8ts.data_ptr(), sis[1:2].data_ptr(), None, ys.data_ptr(), torch.cuda.current_stream().cuda_stream]
    assert L.fp8_linear_fwd(*raw_args) == 0
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(200):
        L.fp8_linear_fwd(*raw_args)
    torch.cuda.synchronize()
    raw_us = (time.perf_counter() - t) / 200 * 1e6
    # the binding's prepared call: checks and marshalling once, then only the C call per call
    prep = F.prepare(small_fwd)
    prep()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(200):
        prep()
    torch.cuda.synchronize()
    prepared_us = (time.perf_counter() - t) / 200 * 1e6
    # the captured graph launched with hipGraphLaunch itself (what a C caller replaying it pays,
    # without torch's replay bookkeeping); the HIP runtime is the one torch already loaded
    hip_graph_us = None
    try:
        hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        hip.hipGraphLaunch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipGraphLaunch.restype = ctypes.c_int
        gexec, gst = int(g.raw_cuda_graph_exec()), torch.cuda.current_stream().cuda_stream
        if hip.hipGraphLaunch(gexec, gst) == 0:
            torch.cuda.synchronize()
            t = time.perf_counter()
            for _ in range(200):
                hip.hipGraphLaunch(gexec, gst)
            torch.cuda.synchronize()
            hip_graph_us = round((time.perf_counter() - t) / 200 * 1e6, 2)
    except (OSError, AttributeError, TypeError, ValueError, RuntimeError):
        pass
    return {"eager_us_per_call": round(eager_us, 2), "graph_replay_us": round(graph_us, 2),
            "c_abi_eager_us_per_call": round(raw_us, 2), "prepared_us_per_call": round(prepared_us, 2),
            "hip_graph_launch_us": hip_graph_us, "launches": 1}


def extras(F, S, torch, np, dev, bf16, step):
    """Timings beyond the step.  The GEMM extras use the step's own FP8 operands (x8, W8, W8^T,
    dy8 cast from the normal-distributed inputs at the step's scales): a GEMM's power draw, and
    with it the clock it runs at, depends on the operands' bits."""
    out = {}
    u8 = dict(device=dev, dtype=torch.uint8)
    f32 = dict(device=dev, dtype=torch.float32)
    flush = torch.empty(512 << 20, **u8)     # 512 MB: evicts the 256 MB MALL and the L2s

    def cold_time(fn, reps=10):
        ts = []
        for _ in range(reps):
            flush.zero_()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e))
        return float(np.median(ts))

    out.update(cast_family(F, S, torch, np, dev, bf16))

    out["small_forward_128x256x256"] = small_forward(F, S, torch, np, dev, bf16)

    # N-chunked GEMM + bias, M=8192, K=N=12288 (x8 and the first 12288 rows of W8), one stream
    # per chunk, captured as one graph
    Mc, Kc, Nc = 8192, 12288, 12288
    A8 = step["x8"]
    B8 = step["w8"][:Nc]
    biasc = bf16(S.normal_bf16(S.seed_for(5, 2), (Nc,), 0.1))
    sa, sb = step["sinv"][0:1], step["sinv"][1:2]
    D = torch.empty((Mc, Nc), device=dev, dtype=torch.bfloat16)
    flop = 2.0 * Mc * Nc * Kc
    graphs = {}
    for nch in (4, 8):
        streams = [torch.cuda.Stream() for _ in range(nch)]
        cap = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        F.fp8_gemm_bias_chunked(A8, 0, sa, B8, 0, sb, biasc, D, nch, streams)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            F.fp8_gemm_bias_chunked(A8, 0, sa, B8, 0, sb, biasc, D, nch, streams, stream=cap)
        g.replay()
        torch.cuda.synchronize()
        graphs[nch] = (g, streams)
    # three rounds, the three forms alternating; each form's best round
    best = {"unchunked": float("inf"), 4: float("inf"), 8: float("inf")}
    for _ in range(3):
        best["unchunked"] = min(best["unchunked"],
                                _time_fn(torch, lambda: F.fp8_gemm_bias(A8, 0, sa, B8, 0, sb, biasc, D), 5))
        for nch in (4, 8):
            best[nch] = min(best[nch], _time_fn(torch, graphs[nch][0].replay, 5))
    res = {"unchunked_tflops": round(flop / (best["unchunked"] * 1e-3) / 1e12, 1),
           "chunks4_graph_tflops": round(flop / (best[4] * 1e-3) / 1e12, 1),
           "chunks8_graph_tflops": round(flop / (best[8] * 1e-3) / 1e12, 1)}
    del graphs
    out["chunked_gemm_8192x12288x12288"] = res
    del A8, B8, D

    # the box's own streaming ceiling: a plain 1 GiB device copy (torch copy_), cold
    src = torch.empty(1 << 30, **u8).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = cold_time(lambda: dst.copy_(src))
    gbps = 2 * (1 << 30) / (ms * 1e-3) / 1e9
    out["copy_1GiB_cold"] = {"us": round(ms * 1e3, 1), "GBps": round(gbps, 1), "frac_hbm": round(gbps * 1e9 / HBM_PEAK, 3)}
    del src, dst

    # lazy transpose-cache fill of FP8 codes, cold (1 B read + 1 B written): the weight
    # [18432, 12288] and the activation [8192, 12288] (seeded random bytes)
    for Rw, Cw in ((18432, 12288), (8192, 12288)):
        W8 = torch.randint(0, 256, (Rw, Cw), generator=torch.Generator().manual_seed(9), dtype=torch.uint8).to(dev)
        nbytes = Rw * Cw * 2
        sets = [(W8 if k == 0 else W8.clone(), torch.empty((Cw, Rw), **u8)) for k in range(_nsets(nbytes))]
        ms = cold_rotating(torch, [lambda a=a, b=b: F.fp8_transpose(a, b) for a, b in sets], nbytes)
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[f"fp8_transpose_{Rw}x{Cw}_cold"] = {"us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                                                 "frac_hbm": round(gbps * 1e9 / HBM_PEAK, 3)}
        del W8, sets

    # GEMM writing an FP8 output with its own scale and amax capture, dgrad shape of the step
    # (M=8192, N=12288, K=18432), against the bfloat16-output GEMM on the same operands
    Mg, Ng, Kg = 8192, 12288, 18432
    A8, B8 = step["dy8"], step["w8t"]      # the dgrad operands: dy8 [M, N] (E5M2), W8^T [K, N]
    sa, sb = step["sinv"][2:3], step["sinv"][1:2]
    D8 = torch.empty((Mg, Ng), **u8)
    Db = torch.empty((Mg, Ng), device=dev, dtype=torch.bfloat16)
    # output scale 2^18: dx ~ N(0, 0.027) here, so its amax lands near the top of E5M2's range
    ds, dsi, dam = torch.tensor([2.0 ** 18], **f32), torch.zeros(1, **f32), torch.zeros(1, **f32)
    flop = 2.0 * Mg * Ng * Kg
    F.fp8_gemm_bias_fp8(A8, F.E5M2, sa, B8, F.E4M3, sb, None, D8, F.E5M2, ds, dsi, dam)
    F.fp8_gemm_bias(A8, F.E5M2, sa, B8, F.E4M3, sb, None, Db)
    torch.cuda.synchronize()
    # alternate the two for three rounds and keep each one's best round, so neither is measured
    # alone in a colder or hotter clock state
    t8 = tb = float("inf")
    for _ in range(3):
        t8 = min(t8, _time_fn(torch, lambda: F.fp8_gemm_bias_fp8(A8, F.E5M2, sa, B8, F.E4M3, sb, None, D8, F.E5M2,
                                                                  ds, dsi, dam), 5))
        tb = min(tb, _time_fn(torch, lambda: F.fp8_gemm_bias(A8, F.E5M2, sa, B8, F.E4M3, sb, None, Db), 5))
    out["fp8_out_gemm_8192x12288x18432"] = {"fp8_out_tflops": round(flop / (t8 * 1e-3) / 1e12, 1),
                                             "bf16_out_tflops": round(flop / (tb * 1e-3) / 1e12, 1)}
    del D8, Db

    # the forward GEMM's speed against its operand bits: the step's own FP8 operands, then the
    # same shapes of zero codes (identical instructions; only the bits the matrix units and data
    # paths toggle differ, and with them the power drawn and the clock the chip holds)
    xz, wz = torch.zeros_like(step["x8"]), torch.zeros_like(step["w8"])
    Mf, Kf = step["x8"].shape
    Nf = step["w8"].shape[0]
    Df = torch.empty((Mf, Nf), device=dev, dtype=torch.bfloat16)
    sx, sw = step["sinv"][0:1], step["sinv"][1:2]
    flop = 2.0 * Mf * Nf * Kf
    tr = tz = float("inf")
    for _ in range(3):
        tr = min(tr, _time_fn(torch, lambda: F.fp8_gemm_bias(step["x8"], F.E4M3, sx, step["w8"], F.E4M3, sw, None, Df), 5))
        tz = min(tz, _time_fn(torch, lambda: F.fp8_gemm_bias(xz, F.E4M3, sx, wz, F.E4M3, sw, None, Df), 5))
    out["gemm_fwd_operand_bits"] = {"step_operands_tflops": round(flop / (tr * 1e-3) / 1e12, 1),
                                    "zero_operands_tflops": round(flop / (tz * 1e-3) / 1e12, 1)}
    del xz, wz, Df

    del flush
    torch.cuda.empty_cache()
    return out


def _host_cores():
    return len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)


def _row_blocks(R, n):
    edges = [R * k // n for k in range(n + 1)]
    return [(a, b) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def _oracle_ct(oracle, x, scale, fmt, nthreads, with_dbias=False):
    """The oracle's cast+transpose (and dbias) of x, one row block per host thread (the ctypes
    calls release the GIL): the blocks' row-major codes stacked, their transposed codes side by
    side, the amax the largest block amax, dbias the sum of the blocks' column sums.  The
    oracle's arithmetic per element is unchanged; only the driver splits the rows."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    def one(ab):
        xb = x[ab[0]:ab[1]]
        q, qt, a, si = oracle.cast_transpose(xb, scale, fmt)
        return q, qt, a, (oracle.dbias(xb) if with_dbias else None)

    blocks = _row_blocks(x.shape[0], nthreads)
    if len(blocks) == 1:
        parts = [one(blocks[0])]
    else:
        with ThreadPoolExecutor(len(blocks)) as ex:
            parts = list(ex.map(one, blocks))
    q = np.concatenate([p[0] for p in parts], 0)
    qt = np.concatenate([p[1] for p in parts], 1)
    amax = max(float(p[2]) for p in parts)
    db = sum(p[3] for p in parts) if with_dbias else None
    return q, qt, amax, db


def _oracle_gemm(oracle, A, fa, sa, B, fb, sb, bias, nthreads):
    """The oracle's float64 GEMM with B split into row blocks (output column blocks), one per
    host thread, each block's product on one BLAS thread; the blocks' outputs side by side."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    blocks = _row_blocks(B.shape[0], nthreads)

    def one(ab):
        return oracle.gemm_bias(A, fa, sa, B[ab[0]:ab[1]], fb, sb, None if bias is None else bias[ab[0]:ab[1]])

    with ThreadPoolExecutor(len(blocks)) as ex:
        return np.concatenate(list(ex.map(one, blocks)), 1)


def cpu_baseline(x_h, w_h, b_h, dy_h):
    """The oracle (as it stands) on the host cores, one thread and threaded over row blocks:
      * the cast family at full size: the small forward layer [128,256] x [256,256] with its
        scale update (all steps), cast+transpose at [1024,1024], [4096,4096], [8192,12288], and
        the backward prep (dbias+cast+transpose of dy [8192,4096], scale update L=1024, T=3);
      * the training step on a bounded sample: 16 of the 8192 token rows of x and dy with the
        full [18432,12288] weight (W cast+transpose at full size, three float64 GEMMs, dbias,
        scale update); `value` is its GEMM FLOP rate with every host core in use.
    A reported baseline only."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synthetic as S

    ncores = _host_cores()
    res = {}

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    # small forward layer (all steps) + its scale update
    xs, ws_, bs = (S.normal_bf16(S.seed_for(0, 0), (128, 256), 1.0), S.normal_bf16(S.seed_for(0, 1), (256, 256), 1.0),
                   S.normal_bf16(S.seed_for(0, 2), (256,), 0.1))

    def small():
        f = oracle.linear_fwd(xs, ws_, bs, 1.0, 1.0, want_x_t=False)
        h = np.zeros((16, 3), np.float32)
        h[0] = [f["x_amax"], f["w_amax"], 0.0]
        oracle.scale_update(h, np.ones(3, np.float32), np.ones(3, np.float32), [0, 0, 1], 0)

    with threadpool_limits(limits=1):
        us_small = min(timed(small) for _ in range(5)) * 1e6
    res["small_forward_128x256x256_us"] = round(us_small, 1)

    # cast+transpose sweep and backward prep at full size, 1 thread and all cores
    sweep = {}
    for idx, (R, C) in enumerate(CT_SHAPES):
        xh = S.outlier_bf16(S.seed_for(1, idx), (R, C), 1.0)
        t1 = timed(lambda: _oracle_ct(oracle, xh, 0.4, 0, 1))
        tn = timed(lambda: _oracle_ct(oracle, xh, 0.4, 0, ncores))
        sweep[f"{R}x{C}"] = {"GBps_1": round(R * C * 4 / t1 / 1e9, 3), "GBps_all": round(R * C * 4 / tn / 1e9, 3)}
    res["cast_transpose_GBps"] = sweep
    R, C = PREP_SHAPE
    dyh = S.normal_bf16(S.seed_for(3, 0), (R, C), 0.01)
    hh = S.log_uniform_f32(S.seed_for(3, 1), 1024 * 3, 1e-3, 1e3).reshape(1024, 3)

    def prep(n):
        _oracle_ct(oracle, dyh, 4096.0, 1, n, with_dbias=True)
        oracle.scale_update(hh, np.ones(3, np.float32), np.ones(3, np.float32), [0, 0, 1], 0)

    t1, tn = timed(lambda: prep(1)), timed(lambda: prep(ncores))
    nb = R * C * 4 + C * 4
    res[f"backward_prep_{R}x{C}_GBps"] = {"GBps_1": round(nb / t1 / 1e9, 3), "GBps_all": round(nb / tn / 1e9, 3)}

    # the training step on 16 token rows with the full weight
    rows = 16
    xs16 = np.ascontiguousarray(x_h[:rows])
    dys16 = np.ascontiguousarray(dy_h[:rows])

    def step_sample(n):
        w8, w8t, w_amax, _ = _oracle_ct(oracle, w_h, 1.0, 0, n)
        w_sinv = oracle.scale_inv(1.0)
        x8, x8t, x_amax, x_sinv = oracle.cast_transpose(xs16, 1.0, 0)
        _oracle_gemm(oracle, x8, 0, x_sinv, w8, 0, w_sinv, b_h, n)                      # forward
        dy8, dy8t, dy_amax, dy_sinv, _ = oracle.dbias_cast_transpose(dys16, 1.0, 1)
        _oracle_gemm(oracle, dy8, 1, dy_sinv, w8t, 0, w_sinv, None, n)                   # dgrad
        _oracle_gemm(oracle, dy8t, 1, dy_sinv, x8t, 0, x_sinv, None, n)                  # wgrad
        h = np.zeros((HIST_L, 3), np.float32)
        h[0] = [x_amax, w_amax, dy_amax]
        oracle.scale_update(h, np.ones(3, np.float32), np.ones(3, np.float32), [0, 0, 1], 0)

    with threadpool_limits(limits=1):
        secn = timed(lambda: step_sample(ncores))
    flop = 3 * 2.0 * rows * N * K
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(flop / secn / 1e12, 6), "unit": "TFLOP/s", "cores": ncores, "kind": "oracle",
            "seconds": round(secn, 2),
            "cast_family": res,
            "cpu_model": model,
            "sample": f"one training step on {rows} of the {M} token rows of x and dy with the full "
                      f"[{N},{K}] weight (W cast+transpose and the three float64 GEMMs split "
                      f"into row blocks, one per host thread; dbias; scale update); FLOPs counted as 3 x 2 x {rows} x {N} x "
                      f"{K}. cast_family: the oracle at full size (GB/s = 4 algorithmic bytes per element / s; "
                      f"_1 one thread, _all one row block per host thread)"}


if __name__ == "__main__":
    main()
