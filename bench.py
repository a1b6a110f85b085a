#!/usr/bin/env python3
"""Benchmark of the blockwise-scaled FP8 GEMM hot path on one MI355X.

Workloads (synthetic, seeded; inputs resident in HBM before timing starts):
  decode   (default) o_proj decode, M=1, N=K=4096.  One step = W8A8 GEMM
           with its 1x128 activation quantisation fused (bf16 activations in)
           + W8A16 GEMM (bf16 activations).  --unfused runs the quantiser as
           its own kernel before the W8A8 GEMM instead.
           Weights rotate over --copies distinct copies so no call finds its
           weights in a cache.  Headline: step HBM GB/s (algorithmic bytes).
  prefill  o_proj prefill, M=N=K=4096, 1% outlier channels.  One step =
           activation quantisation + W8A8 GEMM.  Headline: TFLOP/s.
  blk32    block-32 UE8M0 weight-only GEMM, N=4096, K=7168, M=--m (default 1).
           Headline: HBM GB/s.
  w8a16    W8A16 blk128 GEMM alone, N=K=4096, bf16 activations, M=--m
           (default 4096; M > 16 runs the tiled MFMA kernel).  Headline:
           TFLOP/s against the bf16 MFMA peak (HBM GB/s for M <= 16).
  sweep    W8A8 over the projections (N x K) 4096x4096, 1024x4096, 12288x4096,
           4096x12288 and M in {1, 2, 4, 8, 16, 32, 64, 128, 512, 4096}; weights
           rotate over copies totalling >= 512 MiB per shape.  Per point: GEMM
           and quantiser microseconds and the GEMM's fraction of its roofline
           time max(bytes / 8 TB/s, FLOPs / 5 PFLOP/s).  Headline: geometric
           mean of those fractions.

The timed region runs the K steps kernel by kernel (K back-to-back launches
of each), with one HIP event pair per kernel on the stream the kernels run
on; per-kernel durations are those phase times over K.  The roofline object
reports the dominant kernel's algorithmic bytes (or FLOPs) per launch over
its average duration.  The cpu_baseline object times the CPU oracle on a
bounded sample of the same workload.  For decode, timing.graph also gives
the time per step of one rotation cycle of steps captured as a HIP graph and
replayed (kernels in step order, gaps included, no host launch cost;
--no-graph skips it).

Prints exactly one JSON line on stdout.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs, TFLOP/s, HBM GB/s and % of roofline; blockwise FP8 GEMM N=K=4096, M=1..4096"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", choices=["decode", "prefill", "blk32", "w8a16", "sweep"], default="decode")
    p.add_argument("--m", type=int, default=None, help="token count for blk32 / decode")
    p.add_argument("--copies", type=int, default=24,
                   help="decode: distinct weight copies rotated per kernel (each kernel has its own set); "
                        "other workloads: copies rotated per call")
    p.add_argument("--cpu-seconds", type=float, default=8.0, help="per leg (one thread, all cores)")
    p.add_argument("--no-extras", action="store_true",
                   help="decode: skip the extra kernel lines (read floor, prefill GEMM, block-32 at M = 1)")
    p.add_argument("--sweep-warm-ms", type=float, default=40.0,
                   help="sweep: GPU time each point's GEMM runs back to back before its timed launches")
    p.add_argument("--prefill-warm-ms", type=float, default=250.0,
                   help="GPU time the prefill GEMM runs back to back before its timed launches (clock ramp)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="decode: skip the HIP graph replay timing")
    p.add_argument("--smi", action="store_true",
                   help="record rocm-smi power and clock readings before and after the run in device.smi")
    p.add_argument("--unfused", action="store_true",
                   help="decode: separate quantiser + W8A8 GEMM instead of the fused call")
    p.add_argument("--copy-probe", action="store_true",
                   help="before the workload, copy a 96 MiB buffer 5 times (calibrates HBM byte counters)")
    return p.parse_args()


# ------------------------------------------------------------ byte counts ----
def bytes_quant(M, K):
    G = (K + 127) // 128
    return 2 * M * K + M * K + 4 * M * G


def bytes_w8a8(M, N, K):
    return N * K + 4 * ((N + 127) // 128) * (K // 128) + M * K + 4 * M * ((K + 127) // 128) + 2 * M * N


def bytes_quant_w8a8(M, N, K):
    """Fused quantise + W8A8: 16-bit activations in, no code round trip."""
    return N * K + 4 * ((N + 127) // 128) * (K // 128) + 2 * M * K + 2 * M * N


def bytes_w8a16(M, N, K):
    return N * K + 4 * ((N + 127) // 128) * (K // 128) + 2 * M * K + 2 * M * N


def bytes_blk32(M, N, K):
    return N * K + (N // 32) * (K // 32) + 2 * M * K + 2 * M * N


# ------------------------------------------------- measured HBM traffic ----
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_PROBE_BYTES = 96 << 20


def source_fingerprint():
    """sha256 over the HIP sources and headers the library is built from."""
    import hashlib
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "blockwise_scaled_fp8_amd", "csrc"), os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".hpp", ".h")):
                h.update(name.encode())
                h.update(open(os.path.join(d, name), "rb").read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` in `workload` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE passes, scaled by the copy-kernel
    calibration; None when no such record exists or when the kernel sources
    have changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_fingerprint():
        return None
    k = rec.get("workloads", {}).get(workload, {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def copy_probe(torch):
    a = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


# ------------------------------------------------------------- GPU timing ----
def _sleep_cycles_per_ms(torch):
    """Calibrate torch.cuda._sleep (a spin kernel) in cycles per millisecond."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    a.record()
    torch.cuda._sleep(2_000_000)
    b.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(a.elapsed_time(b), 1e-3)


def run_steps(torch, phases, steps, warmup):
    """Time `steps` steps of the hot path.

    `phases` is an ordered list of (kernel name, launch(i)) pairs; one step is
    one launch of every phase.  The timed region runs the steps phase by phase
    (all `steps` launches of the first kernel, then of the second, ...), which
    is the same work in an order that keeps every data dependency (each phase
    only reads what earlier phases wrote), with one event pair per phase on
    the launch stream.  When the host enqueues a step faster than the GPU runs
    it, a second round of warmup steps is queued right before the timed ones
    (the GPU stays busy from the warmup into the timed region, at the clock the
    warmup reached); otherwise a spin kernel queued right before the timed
    region keeps the GPU busy while the host enqueues every timed launch, so
    the events see back-to-back GPU execution, not host launch latency.
    Returns ms per step and per-kernel average microseconds per launch."""
    t0 = time.perf_counter()
    for i in range(warmup):
        for _, launch in phases:
            launch(i)
    t_host = time.perf_counter() - t0
    torch.cuda.synchronize()
    host_per_step = (time.perf_counter() - t0) / max(warmup, 1)
    enqueue_per_step = t_host / max(warmup, 1)
    # GPU-bound steps (the host enqueues a step in well under the GPU's time
    # for it): the warmup runs straight into the timed region with no idle
    # gap, so the timed steps start at the clock the warmup reached.
    if warmup >= 10 and enqueue_per_step < 0.5 * host_per_step:
        for i in range(warmup):
            for _, launch in phases:
                launch(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
        t_enq = time.perf_counter()
        ev[0].record()
        for p, (_, launch) in enumerate(phases):
            for s in range(steps):
                launch(warmup + s)
            ev[p + 1].record()
        enqueue_ms = (time.perf_counter() - t_enq) * 1e3
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_enq
        kern = {name: {"avg_us": 1e3 * ev[p].elapsed_time(ev[p + 1]) / steps} for p, (name, _) in enumerate(phases)}
        return ev[0].elapsed_time(ev[-1]) / steps, wall, kern, {
            "head_start_ms": 0.0, "host_enqueue_ms": enqueue_ms, "gpu_ahead": True,
            "method": "per-kernel phases of back-to-back launches, HIP events; GPU-bound, so the warmup runs "
                      "straight into the timed region (no idle gap)"}
    cyc_per_ms = _sleep_cycles_per_ms(torch)
    head_ms = 1.5 * host_per_step * steps * 1e3 + 5.0
    for attempt in range(3):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
        torch.cuda.synchronize()
        torch.cuda._sleep(int(head_ms * cyc_per_ms))
        t_enq = time.perf_counter()
        ev[0].record()
        for p, (_, launch) in enumerate(phases):
            for s in range(steps):
                launch(warmup + s)
            ev[p + 1].record()
        enqueue_ms = (time.perf_counter() - t_enq) * 1e3
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_enq
        if enqueue_ms < head_ms:
            break
        head_ms = 2.0 * enqueue_ms + 5.0          # the GPU caught up with the host: retry
    kern = {name: {"avg_us": 1e3 * ev[p].elapsed_time(ev[p + 1]) / steps} for p, (name, _) in enumerate(phases)}
    ms_per_step = ev[0].elapsed_time(ev[-1]) / steps
    return ms_per_step, wall, kern, {"head_start_ms": head_ms, "host_enqueue_ms": enqueue_ms,
                                     "gpu_ahead": enqueue_ms < head_ms,
                                     "method": "per-kernel phases of back-to-back launches, HIP events"}


# ---------------------------------------------------------- cache reuse ----
MALL_BYTES = 256 << 20      # MI355X Infinity Cache (memory-side, shared by all XCDs)


def launch_order(phase_names, copies_of, warmup, steps, gpu_bound_rewarm=True):
    """The (phase, copy) sequence run_steps issues: warmup steps in step
    order (twice when the GPU-bound path queues a second warmup round), then
    the timed steps phase by phase.  Returns the sequence and the position of
    the first timed launch."""
    seq = []
    for _ in range(2 if gpu_bound_rewarm else 1):
        for i in range(warmup):
            seq += [(p, copies_of[p](i)) for p in phase_names]
    timed = len(seq)
    for p in phase_names:
        seq += [(p, copies_of[p](warmup + s)) for s in range(steps)]
    return seq, timed


def min_reuse_bytes(seq, bytes_of, first=0):
    """Smallest number of other weight bytes read between a read at position
    >= `first` in `seq` and the previous read of the same buffer (None when
    no such buffer is read twice)."""
    last, total, best = {}, 0, None
    for pos, (p, c) in enumerate(seq):
        key = (p, c)
        if key in last and pos >= first:
            d = total - last[key]
            best = d if best is None else min(best, d)
        total += bytes_of[p]
        last[key] = total
    return best


def assert_no_cache_reuse(order, bytes_of, what):
    """No timed launch reads a weight copy that less than the last-level
    cache's size of other weights has followed since its previous read."""
    seq, timed = order
    d = min_reuse_bytes(seq, bytes_of, timed)
    assert d is None or d >= MALL_BYTES, (
        f"{what}: a weight copy is re-read after only {d} bytes of other weights (< {MALL_BYTES}, the "
        f"last-level cache): use more copies")
    return d


# ------------------------------------------------------------ CPU baseline ----
def _cpu_share():
    """Host cores this process may use: the affinity mask, capped by the
    thread budget the environment sets (OMP_NUM_THREADS)."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, n)


def _time_calls(fn, seconds):
    calls = 0
    t0 = time.perf_counter()
    while True:
        fn()
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return calls, el


def cpu_baseline(fn, seconds, unit_per_call, unit, sample):
    """The oracle as it stands, timed on the host: once with one BLAS thread
    and once with every core of this process's share; `value` is the
    all-core figure."""
    from threadpoolctl import threadpool_limits
    nproc = len(os.sched_getaffinity(0))
    share = _cpu_share()
    with threadpool_limits(limits=1):
        c1, t1 = _time_calls(fn, seconds)
    with threadpool_limits(limits=share):
        cn, tn = _time_calls(fn, seconds)
    return {"value": unit_per_call * cn / tn, "unit": unit, "cores": share, "kind": "oracle",
            "sample": f"{sample}; {cn} calls in {tn:.1f} s with {share} BLAS threads, {c1} calls in {t1:.1f} s "
                      f"with 1; numpy float64",
            "one_core": {"value": unit_per_call * c1 / t1, "cores": 1}, "nproc": nproc}


# ------------------------------------------------------- extra kernel lines ----
def timed_after_ramp(torch, launch, steps, warm_ms):
    """Run `launch` back to back for about `warm_ms` (the clock ramps up under
    sustained load), then time `steps` more launches with one HIP event pair,
    queued right behind the warm ones.  When the host enqueues a launch more
    slowly than the GPU runs it, a spin kernel queued between the two keeps
    the GPU busy while the host enqueues the timed launches, so the events see
    back-to-back GPU execution rather than the host's launch rate.  Returns
    (us per launch, warm launches, warm ms)."""
    for i in range(5):
        launch(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for i in range(20):
        launch(5 + i)
    b.record()
    host_us = (time.perf_counter() - t0) * 1e6 / 20
    torch.cuda.synchronize()
    est_us = 1e3 * a.elapsed_time(b) / 20
    gpu_bound = host_us < 0.5 * est_us
    cyc_per_ms = None if gpu_bound else _sleep_cycles_per_ms(torch)
    n_warm = max(20, int(warm_ms * 1e3 / max(est_us, host_us, 1e-3)))
    for i in range(n_warm):
        launch(25 + i)
    if not gpu_bound:
        torch.cuda._sleep(int((1.5 * host_us * steps / 1e3 + 2.0) * cyc_per_ms))
    a.record()
    for s in range(steps):
        launch(25 + n_warm + s)
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / steps, n_warm, n_warm * max(est_us, host_us) / 1e3


def read_floor(torch, buffers, nbytes, steps, warmup):
    """Per-launch time of the streaming-read probe over rotated buffers (the
    best of 4, 8 and 16 loads per thread)."""
    import ctypes
    from blockwise_scaled_fp8_amd.build import PROBE_LIB
    lib = ctypes.CDLL(PROBE_LIB)
    lib.bfp8_read_probe.restype = ctypes.c_int
    lib.bfp8_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.bfp8_probe_workgroups.restype = ctypes.c_int64
    lib.bfp8_probe_workgroups.argtypes = [ctypes.c_int64, ctypes.c_int]
    sink = torch.empty(int(lib.bfp8_probe_workgroups(nbytes, 4)), dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = None
    for loads in (4, 8, 16):
        def launch(i, loads=loads):
            rc = lib.bfp8_read_probe(ctypes.c_void_p(buffers[i % len(buffers)].data_ptr()), nbytes, loads,
                                     ctypes.c_void_p(sink.data_ptr()), stream)
            assert rc == 0, rc
        _, _, kern, _ = run_steps(torch, [("read", launch)], steps, warmup)
        us = kern["read"]["avg_us"]
        if best is None or us < best[0]:
            best = (us, loads)
    return {"avg_us": best[0], "alg_bytes": nbytes, "GBps": nbytes / (best[0] * 1e3),
            "hbm_frac": nbytes / (best[0] * 1e3) / HBM_PEAK_GBS, "loads_per_thread": best[1],
            "what": "plain 16-byte streaming read of the same rotated weight copies, one dword written per workgroup; "
                    "best of 4/8/16 loads per thread"}


def extra_prefill(torch, bfp8, inputs, args):
    """The prefill GEMM (M = N = K = 4096, codes in) after the clock has
    ramped: run back to back for --prefill-warm-ms of GPU time first."""
    M = N = K = 4096
    data = inputs.workload(2, M=M)
    xq, xs = bfp8.quantize_act(data["x"].cuda())
    wq, ws = bfp8.quantize_weight(data["w"].cuda())
    copies = [(wq.clone(), ws.clone()) for _ in range(4)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    wsp = bfp8.make_workspace(bfp8.OP_GEMM_W8A8_BLK128, M, N, K)

    def gemm(i):
        a = copies[i % len(copies)]
        bfp8.bfp8_gemm_w8a8_blk128(xq, xs, a[0], a[1], y, wsp)

    us, n_warm, warm_ms = timed_after_ramp(torch, gemm, 200, args.prefill_warm_ms)
    flops = 2.0 * M * N * K
    out = {"avg_us": us, "TFLOPs": flops / (us * 1e6), "mfma_frac": flops / (us * 1e6) / FP8_PEAK_TFLOPS,
           "alg_bytes": bytes_w8a8(M, N, K), "M": M, "N": N, "K": K,
           "kernel": bfp8.bfp8_get_plan(bfp8.OP_GEMM_W8A8_BLK128, M, N, K)["kernel_name"],
           "ramp": f"{n_warm} launches (~{warm_ms:.0f} ms of GPU time) back to back before 200 timed launches, "
                   f"no idle gap: the clock ramps up over the first ~20 ms of sustained load"}
    if args.smi:
        for i in range(int(1000e3 / us)):       # ~1 s of queued work: sample the clock under it
            gemm(i)
        out["smi_under_load"] = smi_sample()
        torch.cuda.synchronize()
    del copies, y, wsp
    return out


def extra_w8a16_tile(torch, bfp8, inputs, args):
    """The W8A16 blk128 GEMM at M = N = K = 4096 (bf16 activations, the
    tiled kernel) after the same clock ramp as the prefill GEMM."""
    M = N = K = 4096
    x = inputs.activations(M, K, workload=2, stream=0, outliers=True).cuda()
    wq, ws = bfp8.quantize_weight(inputs.workload(2)["w"].cuda())
    copies = [(wq.clone(), ws.clone()) for _ in range(4)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    wsb = bfp8.make_workspace(bfp8.OP_GEMM_W8A16_BLK128, M, N, K)

    def gemm(i):
        a = copies[i % len(copies)]
        bfp8.bfp8_gemm_w8a16_blk128(x, a[0], a[1], y, wsb)

    us, n_warm, warm_ms = timed_after_ramp(torch, gemm, 100, args.prefill_warm_ms)
    flops = 2.0 * M * N * K
    del copies, y, wsb
    return {"avg_us": us, "TFLOPs": flops / (us * 1e6), "mfma_frac": flops / (us * 1e6) / BF16_PEAK_TFLOPS,
            "M": M, "N": N, "K": K, "x_dtype": "bf16",
            "kernel": bfp8.bfp8_get_plan(bfp8.OP_GEMM_W8A16_BLK128, M, N, K)["kernel_name"],
            "ramp": f"{n_warm} launches (~{warm_ms:.0f} ms of GPU time) back to back before 100 timed launches"}


def extra_blk32(torch, bfp8, inputs, args, M=1):
    N, K = 4096, 7168
    x = inputs.activations(M, K, workload=3, dtype=torch.float16).cuda()
    wq_h = inputs.block32_codes(N, K, workload=3)
    st, e8_h, bad = bfp8.bfp8_prepare_blk32_ue8m0(wq_h, inputs.block32_scales(N, K, workload=3))
    assert st == 0, (st, bad)
    nb = bytes_blk32(M, N, K)
    ncopy = 12
    copies = [(wq_h.cuda(), e8_h.cuda()) for _ in range(ncopy)]
    assert_no_cache_reuse(launch_order(["g"], {"g": lambda i: i % ncopy}, args.warmup, args.steps), {"g": N * K},
                          "block-32")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    wsb = bfp8.make_workspace(bfp8.OP_GEMM_W8A16_BLK32_UE8M0, M, N, K)

    def gemm(i):
        a = copies[i % ncopy]
        bfp8.bfp8_gemm_w8a16_blk32_ue8m0(x, a[0], a[1], y, wsb)

    _, _, kern, _ = run_steps(torch, [("g", gemm)], args.steps, args.warmup)
    us = kern["g"]["avg_us"]
    # The streaming-read floor over the same rotated weight copies (29 MB a
    # launch, so not the decode line's 16 MiB floor).
    floor = read_floor(torch, [a[0] for a in copies], N * K, args.steps, args.warmup)
    del copies
    return {"avg_us": us, "alg_bytes": nb, "GBps": nb / (us * 1e3), "hbm_frac": nb / (us * 1e3) / HBM_PEAK_GBS,
            "M": M, "N": N, "K": K, "weight_copies": ncopy,
            "kernel": bfp8.bfp8_get_plan(bfp8.OP_GEMM_W8A16_BLK32_UE8M0, M, N, K)["kernel_name"],
            "read_floor_us": floor["avg_us"], "vs_read_floor": us / floor["avg_us"]}


# --------------------------------------------------------------- workloads ----
def graph_timing(torch, phases, steps_per_graph, replays):
    """One rotation cycle of decode steps (every phase of every step, in step
    order) captured as a HIP graph and replayed: the wall-clock time per step
    including the gaps between kernels, with no host launch cost."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(2):
            for _, fn in phases:
                fn(i)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps_per_graph):
            for _, fn in phases:
                fn(i)
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / (replays * steps_per_graph)
    return {"us_per_step": us, "steps_per_replay": steps_per_graph, "replays": replays}


def bench_decode(torch, bfp8, inputs, args):
    M = args.m or 1
    N = K = 4096
    data = inputs.workload(1, M=M)
    x = data["x"].cuda()
    w = data["w"].cuda()
    wq0, ws0 = bfp8.quantize_weight(w)
    # Each kernel rotates over its own set of weight copies, so no copy is
    # read again before more than the last-level cache's size of other
    # weights has streamed through (checked below for the exact launch order).
    C = args.copies
    copies8 = [(wq0.clone(), ws0.clone()) for _ in range(C)]
    copies16 = [(wq0.clone(), ws0.clone()) for _ in range(C)]
    del w
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    y8 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws8 = bfp8.make_workspace(bfp8.OP_GEMM_W8A8_BLK128, M, N, K)
    wsq = bfp8.make_workspace(bfp8.OP_QUANT_GEMM_W8A8_BLK128, M, N, K)
    ws16 = bfp8.make_workspace(bfp8.OP_GEMM_W8A16_BLK128, M, N, K)

    def w8a8(i):
        a = copies8[i % C]
        bfp8.bfp8_gemm_w8a8_blk128(xq, xs, a[0], a[1], y8, ws8)

    def quant_w8a8(i):
        a = copies8[i % C]
        bfp8.bfp8_quant_gemm_w8a8_blk128(x, a[0], a[1], y8, wsq)

    def w8a16(i):
        b = copies16[i % C]
        bfp8.bfp8_gemm_w8a16_blk128(x, b[0], b[1], y16, ws16)

    if args.unfused:
        phases = [("quant_act_1x128", lambda i: bfp8.bfp8_quantize_act_1x128(x, xq, xs)),
                  ("gemm_w8a8_blk128", w8a8), ("gemm_w8a16_blk128", w8a16)]
    else:
        phases = [("quant_gemm_w8a8_blk128", quant_w8a8), ("gemm_w8a16_blk128", w8a16)]
    names = [n for n, _ in phases]
    set_of = {"quant_act_1x128": None, "gemm_w8a8_blk128": "w8", "quant_gemm_w8a8_blk128": "w8",
              "gemm_w8a16_blk128": "w16"}
    weight_phases = [n for n in names if set_of[n]]
    seq, timed = launch_order(weight_phases, {n: (lambda i: i % C) for n in weight_phases}, args.warmup, args.steps)
    seq = [(set_of[p], c) for p, c in seq]
    reuse = assert_no_cache_reuse((seq, timed), {"w8": N * K, "w16": N * K}, "decode")
    ms, wall, kern, timing = run_steps(torch, phases, args.steps, args.warmup)
    nbytes = {"quant_act_1x128": bytes_quant(M, K), "gemm_w8a8_blk128": bytes_w8a8(M, N, K),
              "quant_gemm_w8a8_blk128": bytes_quant_w8a8(M, N, K), "gemm_w8a16_blk128": bytes_w8a16(M, N, K)}
    nbytes = {n: nbytes[n] for n in names}
    for n in names:
        kern[n]["alg_bytes"] = nbytes[n]
        kern[n]["GBps"] = nbytes[n] / (kern[n]["avg_us"] * 1e3)
        kern[n]["hbm_frac"] = kern[n]["GBps"] / HBM_PEAK_GBS
    step_bytes = sum(nbytes.values())
    dom = max([n for n in names if n != "quant_act_1x128"], key=lambda n: kern[n]["avg_us"])
    roof = {"kernel": dom, "bound": "hbm", "achieved": kern[dom]["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": kern[dom]["GBps"] / HBM_PEAK_GBS, "traffic": measured_traffic("decode_unfused" if args.unfused else "decode", dom),
            "alg_bytes": nbytes[dom]}
    result = {"value": step_bytes / (ms * 1e6), "unit": "GB/s", "ms_per_step": ms, "dtype": "e4m3,bf16",
              "config": {"workload": ("o_proj decode: 1x128 act quant + W8A8 blk128 + W8A16 blk128 (bf16 x)"
                                      if args.unfused else
                                      "o_proj decode: W8A8 blk128 with fused 1x128 act quant + W8A16 blk128 (bf16 x)"),
                         "M": M, "N": N, "K": K, "weight_copies": 2 * C, "out_dtype": "bf16",
                         "step_alg_bytes": step_bytes},
              "roofline": roof, "kernels": kern, "wall_s": wall, "timing": timing}
    result["timing"]["weight_rotation"] = (
        f"{C} copies per GEMM kernel ({2 * C} in all, 16 MiB each); fewest other weight bytes between two reads "
        f"of one copy in this run's launch order: {reuse} (last-level cache {MALL_BYTES})")

    if not args.no_graph:
        result["timing"]["graph"] = graph_timing(torch, phases, C, max(1, args.steps // C))

    if not args.no_extras:
        floor = read_floor(torch, [a[0] for a in copies8], N * K, args.steps, args.warmup)
        for n in names:
            if set_of[n]:
                kern[n]["vs_read_floor"] = kern[n]["avg_us"] / floor["avg_us"]
        kern["read_floor"] = floor
        kern["prefill_gemm_w8a8_blk128"] = extra_prefill(torch, bfp8, inputs, args)
        kern["w8a16_tile_m4096"] = extra_w8a16_tile(torch, bfp8, inputs, args)
        torch.cuda.empty_cache()
        kern["blk32_m1"] = extra_blk32(torch, bfp8, inputs, args, M=1)
        kern["blk32_m16"] = extra_blk32(torch, bfp8, inputs, args, M=16)

    if not args.no_cpu_baseline:
        import oracle
        xh = data["x"].float().numpy()
        wq_h, ws_h = wq0.cpu().numpy(), ws0.cpu().numpy()

        def one():
            q, s = oracle.quantize_act_1x128(xh)
            oracle.gemm_w8a8_blk128(q, s, wq_h, ws_h)
            oracle.gemm_w8a16_blk128(xh, wq_h, ws_h)

        result["cpu_baseline"] = cpu_baseline(one, args.cpu_seconds, step_bytes / 1e9, "GB/s",
                                              f"full decode step (M={M}, N=K=4096) repeated")
    return result


def bench_prefill(torch, bfp8, inputs, args):
    M = args.m or 4096
    N = K = 4096
    data = inputs.workload(2, M=M)
    x = data["x"].cuda()
    wq, ws = bfp8.quantize_weight(data["w"].cuda())
    copies = [(wq.clone(), ws.clone()) for _ in range(4)]
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    wsp = bfp8.make_workspace(bfp8.OP_GEMM_W8A8_BLK128, M, N, K)

    def gemm(i):
        a = copies[i % len(copies)]
        bfp8.bfp8_gemm_w8a8_blk128(xq, xs, a[0], a[1], y, wsp)

    phases = [("quant_act_1x128", lambda i: bfp8.bfp8_quantize_act_1x128(x, xq, xs)), ("gemm_w8a8_blk128", gemm)]
    ms, wall, kern, timing = run_steps(torch, phases, args.steps, args.warmup)
    flops = 2.0 * M * N * K
    kern["quant_act_1x128"]["alg_bytes"] = bytes_quant(M, K)
    kern["quant_act_1x128"]["GBps"] = bytes_quant(M, K) / (kern["quant_act_1x128"]["avg_us"] * 1e3)
    g = kern["gemm_w8a8_blk128"]
    g["alg_bytes"] = bytes_w8a8(M, N, K)
    g["TFLOPs"] = flops / (g["avg_us"] * 1e6)
    roof = {"kernel": "gemm_w8a8_blk128", "bound": "mfma", "achieved": g["TFLOPs"], "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": g["TFLOPs"] / FP8_PEAK_TFLOPS,
            "traffic": measured_traffic("prefill", "gemm_w8a8_blk128"), "alg_bytes": g["alg_bytes"]}
    result = {"value": flops / (ms * 1e9), "unit": "TFLOP/s", "ms_per_step": ms, "dtype": "e4m3",
              "config": {"workload": "o_proj prefill: 1x128 act quant + W8A8 blk128, 1% outlier channels",
                         "M": M, "N": N, "K": K, "out_dtype": "bf16"},
              "roofline": roof, "kernels": kern, "wall_s": wall, "timing": timing}
    if not args.no_cpu_baseline:
        import oracle
        rows = 8
        xh = data["x"][:rows].float().numpy()
        wq_h, ws_h = wq.cpu().numpy(), ws.cpu().numpy()

        def one():
            q, s = oracle.quantize_act_1x128(xh)
            oracle.gemm_w8a8_blk128(q, s, wq_h, ws_h)

        result["cpu_baseline"] = cpu_baseline(one, args.cpu_seconds, 2.0 * rows * N * K / 1e12, "TFLOP/s",
                                              f"{rows} of {M} token rows of the prefill step")
    return result


def bench_blk32(torch, bfp8, inputs, args):
    M = args.m or 1
    N, K = 4096, 7168
    x = inputs.activations(M, K, workload=3, dtype=torch.float16).cuda()
    wq_h = inputs.block32_codes(N, K, workload=3)
    s_h = inputs.block32_scales(N, K, workload=3)
    st, e8_h, bad = bfp8.bfp8_prepare_blk32_ue8m0(wq_h, s_h)
    assert st == 0, (st, bad)
    copies = [(wq_h.cuda(), e8_h.cuda()) for _ in range(args.copies)]
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    wsb = bfp8.make_workspace(bfp8.OP_GEMM_W8A16_BLK32_UE8M0, M, N, K)

    def gemm(i):
        a = copies[i % len(copies)]
        bfp8.bfp8_gemm_w8a16_blk32_ue8m0(x, a[0], a[1], y, wsb)

    names = ["gemm_w8a16_blk32_ue8m0"]
    ms, wall, kern, timing = run_steps(torch, [(names[0], gemm)], args.steps, args.warmup)
    nb, flops = bytes_blk32(M, N, K), 2.0 * M * N * K
    k = kern[names[0]]
    k["alg_bytes"] = nb
    k["GBps"] = nb / (k["avg_us"] * 1e3)
    k["TFLOPs"] = flops / (k["avg_us"] * 1e6)
    # Up to one 16-token tile the weights bound it (HBM); above, the fp16
    # matrix core (the same split as the W8A16 blk128 line).
    if M <= 16:
        roof = {"kernel": names[0], "bound": "hbm", "achieved": k["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": k["GBps"] / HBM_PEAK_GBS, "traffic": measured_traffic(f"blk32_m{M}", names[0]),
                "alg_bytes": nb}
        value, unit = nb / (ms * 1e6), "GB/s"
    else:
        roof = {"kernel": names[0], "bound": "mfma", "achieved": k["TFLOPs"], "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": k["TFLOPs"] / BF16_PEAK_TFLOPS, "traffic": None, "alg_bytes": nb}
        value, unit = flops / (ms * 1e9), "TFLOP/s"
    result = {"value": value, "unit": unit, "ms_per_step": ms, "dtype": "f16",
              "config": {"workload": "block-32 UE8M0 W8A16 GEMM, fp16 x and out", "M": M, "N": N, "K": K,
                         "weight_copies": len(copies)},
              "roofline": roof, "kernels": kern, "wall_s": wall, "timing": timing}
    if not args.no_cpu_baseline:
        import oracle
        rows = min(M, 8)
        xh = x[:rows].float().cpu().numpy()
        wqn, e8n = wq_h.numpy(), e8_h.numpy()
        result["cpu_baseline"] = cpu_baseline(lambda: oracle.gemm_w8a16_blk32_ue8m0(xh, wqn, e8n), args.cpu_seconds,
                                              2.0 * rows * N * K / 1e12 if M > 16 else bytes_blk32(rows, N, K) / 1e9,
                                              unit, f"{rows} of {M} token rows")
    return result


def bench_w8a16(torch, bfp8, inputs, args):
    M = args.m or 4096
    N = K = 4096
    x = inputs.activations(M, K, workload=2, stream=0, outliers=True).cuda()
    wq, ws = bfp8.quantize_weight(inputs.workload(2)["w"].cuda())
    # Up to M = 256 the weights dominate the traffic: rotate 32 copies (512 MB)
    # so that no call finds its weights in the 256 MB last-level cache.
    ncopy = 32 if M <= 256 else 4
    copies = [(wq.clone(), ws.clone()) for _ in range(ncopy)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    wsb = bfp8.make_workspace(bfp8.OP_GEMM_W8A16_BLK128, M, N, K)

    def gemm(i):
        a = copies[i % len(copies)]
        bfp8.bfp8_gemm_w8a16_blk128(x, a[0], a[1], y, wsb)

    name = "gemm_w8a16_blk128"
    ms, wall, kern, timing = run_steps(torch, [(name, gemm)], args.steps, args.warmup)
    k = kern[name]
    nb, flops = bytes_w8a16(M, N, K), 2.0 * M * N * K
    k["alg_bytes"], k["TFLOPs"], k["GBps"] = nb, flops / (k["avg_us"] * 1e6), nb / (k["avg_us"] * 1e3)
    if M <= 16:
        roof = {"kernel": name, "bound": "hbm", "achieved": k["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": k["GBps"] / HBM_PEAK_GBS, "traffic": None, "alg_bytes": nb}
        value, unit = nb / (ms * 1e6), "GB/s"
    else:
        roof = {"kernel": name, "bound": "mfma", "achieved": k["TFLOPs"], "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": k["TFLOPs"] / BF16_PEAK_TFLOPS, "traffic": None, "alg_bytes": nb}
        value, unit = flops / (ms * 1e9), "TFLOP/s"
    result = {"value": value, "unit": unit, "ms_per_step": ms, "dtype": "e4m3,bf16",
              "config": {"workload": "W8A16 blk128 GEMM, bf16 x with 1% outlier channels", "M": M, "N": N, "K": K,
                         "weight_copies": ncopy, "out_dtype": "bf16"},
              "roofline": roof, "kernels": kern, "wall_s": wall, "timing": timing}
    if not args.no_cpu_baseline:
        import oracle
        rows = min(M, 8)
        xh = x[:rows].float().cpu().numpy()
        wq_h, ws_h = wq.cpu().numpy(), ws.cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(lambda: oracle.gemm_w8a16_blk128(xh, wq_h, ws_h), args.cpu_seconds,
                                              2.0 * rows * N * K / (1e12 if M > 16 else 1.0) if M > 16 else
                                              bytes_w8a16(rows, N, K) / 1e9, unit, f"{rows} of {M} token rows")
    return result


def cases_variant(bfp8, M, N, K):
    p = bfp8.bfp8_get_plan(bfp8.OP_GEMM_W8A8_BLK128, M, N, K)
    v = p["kernel_name"]
    if "tile" in v or "wide" in v:
        v += f":{p['tile_n']}x{p['tile_m']}w{p['waves']}"
    return v + (f"/split{p['splits']}" if p["splits"] > 1 else "")


def bench_sweep(torch, bfp8, inputs, args):
    import math
    points = []
    steps = max(10, min(args.steps, 50))
    for (N, K) in inputs.SWEEP_SHAPES:
        w = inputs.weights_bf16(N, K, workload=4, stream=N + K).cuda()
        wq0, ws0 = bfp8.quantize_weight(w)
        del w
        ncopy = max(2, min(64, -(-(512 << 20) // (N * K))))
        copies = [(wq0.clone(), ws0.clone()) for _ in range(ncopy)]
        for M in inputs.SWEEP_M:
            x = inputs.activations(M, K, workload=4, stream=M).cuda()
            xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
            xs = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            wsb = bfp8.make_workspace(bfp8.OP_GEMM_W8A8_BLK128, M, N, K)

            def gemm(i, copies=copies, xq=xq, xs=xs, y=y, wsb=wsb):
                a = copies[i % len(copies)]
                bfp8.bfp8_gemm_w8a8_blk128(xq, xs, a[0], a[1], y, wsb)

            phases = [("quant_act_1x128", lambda i, x=x, xq=xq, xs=xs: bfp8.bfp8_quantize_act_1x128(x, xq, xs))]
            _, _, kern, _ = run_steps(torch, phases, steps, max(3, args.warmup))
            bfp8.bfp8_quantize_act_1x128(x, xq, xs)
            # The GEMM after a time-based ramp (the clock needs ~20 ms of load),
            # rotating over the copies from the first launch on.
            g_us, _, _ = timed_after_ramp(torch, gemm, steps, args.sweep_warm_ms)
            nbytes, flops = bytes_w8a8(M, N, K), 2.0 * M * N * K
            roof_us = max(nbytes / (HBM_PEAK_GBS * 1e3), flops / (FP8_PEAK_TFLOPS * 1e6))
            points.append({"N": N, "K": K, "M": M, "kernel": cases_variant(bfp8, M, N, K),
                           "gemm_us": g_us, "quant_us": kern["quant_act_1x128"]["avg_us"],
                           "TFLOPs": flops / (g_us * 1e6), "GBps": nbytes / (g_us * 1e3),
                           "bound": "hbm" if nbytes / (HBM_PEAK_GBS * 1e3) >= flops / (FP8_PEAK_TFLOPS * 1e6) else "mfma",
                           "roofline_frac": roof_us / g_us, "copies": len(copies)})
            print(json.dumps(points[-1]), file=sys.stderr, flush=True)
            del x, xq, xs, y, wsb
        del copies
        torch.cuda.empty_cache()
    geo = math.exp(sum(math.log(p["roofline_frac"]) for p in points) / len(points))
    worst = min(points, key=lambda p: p["roofline_frac"])
    return {"value": geo, "unit": "fraction of roofline (geometric mean)", "ms_per_step": sum(p["gemm_us"] for p in points) / 1e3,
            "dtype": "e4m3",
            "config": {"workload": "W8A8 projection sweep (N x K) x M", "shapes": [list(s) for s in inputs.SWEEP_SHAPES],
                       "M": list(inputs.SWEEP_M), "steps_per_point": steps},
            "roofline": {"kernel": "gemm_w8a8_blk128", "bound": worst["bound"], "achieved": worst["roofline_frac"],
                         "peak": 1.0, "unit": "fraction", "frac": worst["roofline_frac"], "traffic": None,
                         "note": "worst point of the sweep"},
            "kernels": {"points": points},
            "timing": {"method": f"GEMM: back-to-back launches for ~{args.sweep_warm_ms:.0f} ms of GPU time, then "
                                 f"the timed ones with no gap (HIP events); quantiser: per-kernel phases"}}


def smi_sample():
    """Power and clock readings of the GPU from rocm-smi (a child process), or
    the reason there are none."""
    import subprocess
    try:
        p = subprocess.run(["rocm-smi", "--showpower", "--showclocks", "--json"], stdout=subprocess.PIPE,
                           stderr=subprocess.PIPE, text=True, timeout=30)
        data = json.loads(p.stdout)
    except Exception as e:   # tool missing, refused or unparsable: say so instead
        return {"error": f"{type(e).__name__}: {e}"[:200]}
    out = {}
    for card, vals in data.items():
        if isinstance(vals, dict):
            out[card] = {k: v for k, v in vals.items() if any(w in k.lower() for w in ("power", "clk", "clock"))}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    import blockwise_scaled_fp8_amd as bfp8
    from blockwise_scaled_fp8_amd import inputs
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    bfp8.load()
    if args.copy_probe:
        copy_probe(torch)
    fn = {"decode": bench_decode, "prefill": bench_prefill, "blk32": bench_blk32, "w8a16": bench_w8a16,
          "sweep": bench_sweep}[args.workload]
    smi_before = smi_sample() if args.smi else None
    r = fn(torch, bfp8, inputs, args)
    device = {"name": torch.cuda.get_device_name(0),
              "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", ""),
              "compute_units": torch.cuda.get_device_properties(0).multi_processor_count}
    if args.smi:
        device["smi"] = {"before": smi_before, "after": smi_sample()}
    line = {"metric": METRIC, "value": r["value"], "unit": r["unit"], "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": r["dtype"], "data": "synthetic", "config": r["config"],
            "roofline": r["roofline"], "cpu_baseline": r.get("cpu_baseline"), "kernels": r["kernels"],
            "timing": r["timing"], "device": device}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
