#!/usr/bin/env python3
"""Throughput of the W4A16 linear forward (awq_gemm) on one MI355X.

Headline workload (the decode target): M=1, K=8192, N=7168, group_size=128,
no bias -- one awq_gemm call per step, algorithmic bytes per step =
qweight + qzeros + scales + x + y.  The metric also names prefill TFLOP/s; the
prefill fused-QKV workload (M=2048, K=4096, N=12288, group_size=128, bias) is
measured in the same run and reported under "prefill" on the same line.

Timing: inputs are resident in HBM before the timed region.  The weights,
zeros, scales, x and y of each step rotate through enough distinct copies to
exceed twice the 256 MiB Infinity Cache, so every step streams its weights
from HBM.  W warmup steps, then exactly K steps recorded in a HIP graph and
replayed once between device synchronisations (this removes host launch
gaps, which are comparable to a decode kernel's duration).  Right before the
timed replay the same graph is replayed untimed for about 20 ms, enqueued
back to back with it, so that the K timed steps run at the clocks of
continuous work however few they are (`untimed_settle_ms` on the line).  HIP
events on the launching stream bracket the timed replay; since the graph runs
one kernel per step back to back, the replay time per step is the kernel's
average duration and the roofline figures use it (it agrees with rocprofv3's
kernel durations).  Events around single launches are reported as well, for
reference.

Prints one JSON line on stdout.  --gpus above 1 is refused: this build is the
single-GPU share of the path.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix cores
ROTATE_BYTES = 512 << 20        # two Infinity Caches

DECODE = dict(workload="decode_m1_k8192_n7168_g128", source="decode_sweep_k8192_n7168",
              M=1, group_size=128)
PREFILL = dict(workload="prefill_qkv_m2048_k4096_n12288_g128",
               source="prefill_qkv_m2048_k4096_n12288", M=2048, group_size=128)


def measured_traffic(leg):
    """HBM-side bytes per launch of the leg's kernel from the committed PMC
    measurement (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE, calibrated
    on a plain copy), or None when the kernel's sources changed since."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            entry = json.load(f)[leg]
        h = hashlib.sha256()
        for fn in entry["sources"]:
            with open(os.path.join(ROOT, fn), "rb") as f:
                h.update(f.read())
        return entry["bytes_per_launch"] if h.hexdigest() == entry["sources_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def algorithmic_bytes(M, K, N, G, bias):
    """qweight + qzeros + scales + x + y (+ bias), each read or written once."""
    return K * N // 2 + G * N // 2 + G * N * 2 + M * K * 2 + M * N * 2 + (2 * N if bias else 0)


def problem_dims(p):
    K = p["qweight"].shape[0]
    N = p["qweight"].shape[1] * 8
    G = p["qzeros"].shape[0]
    return K, N, G


def make_copies(torch, p, R, dev):
    base = {k: torch.from_numpy(v).to(dev) for k, v in p.items()
            if k in ("qweight", "qzeros", "scales", "x")}
    bias = torch.from_numpy(p["bias"]).to(dev) if p["bias"] is not None else None
    M = p["x"].shape[0]
    _, N, _ = problem_dims(p)
    copies = []
    for _ in range(R):
        c = {k: v.clone() for k, v in base.items()}
        c["bias"] = bias
        c["y"] = torch.empty((M, N), dtype=torch.float16, device=dev)
        copies.append(c)
    return copies


# Timed work per point when the step count is left to run_leg: a graph
# replay of a few milliseconds reads 10-18 % slow (the clocks are still
# rising after the set-up pauses: K = 4096, N = 12288, M = 2048 took 206-217
# us per call over 20 calls, 181-184 us over 100-500, on one box), so every
# timed region lasts about this long.
TIMED_SECONDS = 0.05


# Before every timed graph replay the same graph is replayed untimed for
# about this long, enqueued back to back with the timed replay (no host
# synchronisation in between), so that the timed steps run at the clocks of
# continuous work whatever their number.  Without it a 20-step region right
# after a synchronisation read 9 % slow at decode (10.66 against 9.78 us per
# call) and 15 % at the prefill projection (210.5 against 178-184 us).
SETTLE_SECONDS = 0.02


def settled_replay_ms(torch, graph, stream, calls):
    """Replays `graph` (already uploaded) untimed for about SETTLE_SECONDS,
    then once more between HIP events on `stream`; returns (ms of the timed
    replay, ms spent settling).  The caller synchronises before and after."""
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    with torch.cuda.stream(stream):
        graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    probe_ms = max(t0.elapsed_time(t1), 1e-3)
    n = int(min(10000, -(-SETTLE_SECONDS * 1e3 // probe_ms)))
    with torch.cuda.stream(stream):
        for _ in range(n):
            graph.replay()
    t0.record(stream)
    with torch.cuda.stream(stream):
        graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1), n * probe_ms


def auto_steps(nbytes, nflops):
    """Steps for about TIMED_SECONDS of timed work: the call's time
    estimated from half the HBM and matrix-core peaks, 50 to 2000 steps."""
    est = max(nbytes / (HBM_PEAK_GBS * 0.5e9), nflops / (FP16_MFMA_PEAK_TFLOPS * 0.4e12), 5e-6)
    return int(min(2000, max(50, -(-TIMED_SECONDS // est))))


def run_leg(torch, awq, spec, steps, warmup, dev, events=True, eager=True):
    """One workload point timed (steps=None: auto_steps)."""
    import awq_inputs
    p = awq_inputs.workload_inputs(spec["source"], spec["M"], spec["group_size"])
    M = spec["M"]
    g = spec["group_size"]
    K, N, G = problem_dims(p)
    nbytes = algorithmic_bytes(M, K, N, G, p["bias"] is not None)
    nflops = 2 * M * N * K
    if steps is None:
        steps = auto_steps(nbytes, nflops)
    act = spec.get("gidx")   # None, "act_order" or "uneven"
    if act:
        # The same weight under a row-to-group map: g_idx (K int32) is read
        # by the method too; the load-time rebuild is not timed.
        nbytes += 4 * K
    R = max(2, -(-ROTATE_BYTES // nbytes))
    copies = make_copies(torch, p, R, dev)
    ws_bytes = awq.gemm_workspace_size(M, K, N, g)
    path, need = awq.gemm_plan(M, K, N, g, copies[0]["x"].data_ptr(),
                               copies[0]["scales"].data_ptr())
    assert need <= ws_bytes
    if act:
        g_idx = (awq_inputs.act_order_g_idx(K, g, seed=K + N) if act == "act_order"
                 else awq_inputs.random_g_idx(K, G, seed=K + N))
        for c in copies:
            c["w"] = awq.prepare_gidx(c["qweight"], c["qzeros"], c["scales"], g_idx)
            del c["qweight"], c["qzeros"], c["scales"]
        w0 = copies[0]["w"]
        ws_bytes = awq.sorted_workspace_size(M, w0.rows, N, w0.block_rows)
        path, _ = awq.gemm_plan(M, w0.rows, N, w0.block_rows)
        p = dict(p, g_idx=g_idx)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step(i):
        c = copies[i % R]
        if act:
            awq.gemm_sorted(c["x"], c["w"], c["bias"], out=c["y"], workspace=ws)
        else:
            awq.gemm(c["x"], c["qweight"], c["qzeros"], c["scales"], c["bias"], g, out=c["y"],
                     workspace=ws)

    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    torch.cuda.synchronize()

    # Single launches: HIP events around each launch, on the launching stream.
    kern_ms = [float("nan")]
    if events:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        with torch.cuda.stream(stream):
            for i in range(steps):
                ev[i][0].record(stream)
                step(i)
                ev[i][1].record(stream)
        torch.cuda.synchronize()
        kern_ms = [a.elapsed_time(b) for a, b in ev]
    kern_avg_ms = statistics.fmean(kern_ms)

    # Whole job: exactly `steps` steps captured in one graph, replayed once.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    graph.replay()                      # first replay uploads the graph
    torch.cuda.synchronize()
    total_ms, settle_ms = settled_replay_ms(torch, graph, stream, steps)
    ms_per_step = total_ms / steps

    # Eager loop for reference (host launch overhead included), from an idle
    # GPU, between HIP events: the time per call is the slower of the host's
    # launch path and the kernel.  At least ~20 ms of calls, so that the
    # clocks' rise at the start is a small share.
    eager_ms = float("nan")
    if eager:
        n_eager = max(steps, int(-(-SETTLE_SECONDS // max(ms_per_step * 1e-3, 1e-7))))
        n_eager = min(n_eager, 5000)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        with torch.cuda.stream(stream):
            for i in range(n_eager):
                step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / n_eager
    del graph

    sorted_rows = copies[0]["w"].rows if act else K
    return dict(p=p, M=M, K=K, N=N, G=G, g=g, nbytes=nbytes, nflops=nflops, R=R,
                sorted_rows=sorted_rows, steps=steps, settle_ms=settle_ms,
                path=awq.PATH_NAMES[path], ms_per_step=ms_per_step, kern_avg_ms=kern_avg_ms,
                kern_min_ms=min(kern_ms), eager_ms=eager_ms, ws_bytes=ws_bytes)


# Every seeded workload point, in the order the workloads are listed, with
# a short label: c0 tiny, c1 decode N=1280, c2 decode batch sweep, c3 the
# prefill projection, c4 the down-projection at both group sizes.
CONFIG_POINTS = (
    [("c0", "tiny_m4_k256_n128", 4, 64), ("c1", "decode_k8192_n1280", 1, 128)]
    + [("c2", "decode_sweep_k8192_n7168", M, 128) for M in (1, 4, 8, 16)]
    + [("c3", "prefill_qkv_m2048_k4096_n12288", 2048, 128)]
    + [("c4", "mlp_down_k14336_n4096", M, g) for g in (128, -1) for M in (1, 16, 256, 1024, 4096)]
)


def binding_roof(nbytes, nflops, sec):
    """(bound, fraction of that roof): whichever of HBM bytes and matrix-core
    flops takes longer at peak binds the point."""
    gbs = nbytes / sec / 1e9
    tfs = nflops / sec / 1e12
    hbm = nbytes / HBM_PEAK_GBS >= nflops / FP16_MFMA_PEAK_TFLOPS / 1e3
    return ("hbm", gbs / HBM_PEAK_GBS) if hbm else ("mfma", tfs / FP16_MFMA_PEAK_TFLOPS)


def config_points(torch, awq, dev):
    """Each seeded point timed like the headline legs (graph replay, weights
    rotated past the last-level cache, about TIMED_SECONDS of timed work),
    against its binding roof."""
    out = []
    for label, name, M, g in CONFIG_POINTS:
        print(f"[bench] config {label} {name} M={M} g={g}", file=sys.stderr, flush=True)
        r = run_leg(torch, awq, dict(source=name, M=M, group_size=g), None, 5, dev,
                    events=False, eager=False)
        sec = r["ms_per_step"] * 1e-3
        bound, frac = binding_roof(r["nbytes"], r["nflops"], sec)
        out.append({"config": label, "M": M, "K": r["K"], "N": r["N"], "g": g,
                    "kernel": r["path"], "us": round(sec * 1e6, 3), "steps": r["steps"],
                    "GB_per_s": round(r["nbytes"] / sec / 1e9, 1),
                    "TFLOP_per_s": round(r["nflops"] / sec / 1e12, 2),
                    "bound": bound, "frac": round(frac, 4)})
        del r
        torch.cuda.empty_cache()
    return out


def graph_time_us(torch, fn, calls, dev):
    """Per-call time of fn(i) for i < calls, captured in one graph and
    replayed once between HIP events on the capturing stream."""
    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        for i in range(3):
            fn(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(calls):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    ms, _ = settled_replay_ms(torch, graph, stream, calls)
    del graph
    return ms * 1e3 / calls


def read_stream_fn(torch, bufs, dev):
    """A launcher of the plain read-stream kernel (libawq_bench.so, a
    measurement aid built beside the library) over bufs[i % len(bufs)]."""
    import ctypes
    from bit_weight_quantized_awq_amd import build as _build
    lib = ctypes.CDLL(_build.BENCH_LIB_PATH)
    lib.awq_bench_read_stream.restype = ctypes.c_int
    lib.awq_bench_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    nbytes = bufs[0].numel() * bufs[0].element_size()

    def fn(i):
        st = lib.awq_bench_read_stream(bufs[i % len(bufs)].data_ptr(), nbytes, sink.data_ptr(),
                                       1024, torch._C._cuda_getCurrentRawStream(dev.index))
        if st != 0:
            raise RuntimeError(f"awq_bench_read_stream: status {st}")
    return fn


def empty_launch_fn(torch, dev, blocks, threads):
    """A launcher of a kernel that does nothing (libawq_bench.so), with the
    decode kernel's grid shape: the per-call floor of a graph replay."""
    import ctypes
    from bit_weight_quantized_awq_amd import build as _build
    lib = ctypes.CDLL(_build.BENCH_LIB_PATH)
    lib.awq_bench_empty.restype = ctypes.c_int
    lib.awq_bench_empty.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def fn(i):
        st = lib.awq_bench_empty(sink.data_ptr(), blocks, threads,
                                 torch._C._cuda_getCurrentRawStream(dev.index))
        if st != 0:
            raise RuntimeError(f"awq_bench_empty: status {st}")
    return fn


def same_box_references(torch, dev, decode_bytes):
    """What this box does, in this process, on plain work of the headline
    sizes: a read-only stream (a plain kernel of 1024 work-groups, eight
    16-byte loads in flight per thread) and a device copy over the decode
    step's byte count (rounded down to 16 bytes), rotated like the decode
    leg; a kernel that does nothing, launched with the decode grid (what
    one launch costs per call of a graph replay); and torch's float16
    linear (the vendor GEMM) at the prefill projection's shape."""
    n = decode_bytes // 16 * 4
    R = max(2, -(-ROTATE_BYTES // decode_bytes))
    gen = torch.Generator(device="cpu").manual_seed(7)
    bufs = [torch.randint(-2**31, 2**31 - 1, (n,), generator=gen, dtype=torch.int32).to(dev)
            for _ in range(R)]
    dst = [torch.empty_like(b) for b in bufs]
    read_us = graph_time_us(torch, read_stream_fn(torch, bufs, dev), auto_steps(n * 4, 0), dev)
    empty_us = graph_time_us(torch, empty_launch_fn(torch, dev, 448, 256), 2000, dev)
    copy_us = graph_time_us(torch, lambda i: dst[i % R].copy_(bufs[i % R]),
                            auto_steps(2 * n * 4, 0), dev)
    del bufs, dst
    torch.cuda.empty_cache()
    M, K, N = 2048, 4096, 12288
    x = torch.randn((M, K), generator=gen).to(torch.float16).to(dev)
    ws = [(torch.randn((N, K), generator=gen) * 0.02).to(torch.float16).to(dev) for _ in range(2)]
    b = (torch.randn((N,), generator=gen) * 0.1).to(torch.float16).to(dev)
    lin_us = graph_time_us(torch, lambda i: torch.nn.functional.linear(x, ws[i % 2], b),
                           auto_steps(2 * N * K, 2 * M * N * K), dev)
    del x, ws, b
    torch.cuda.empty_cache()
    return {
        "read_stream": {"op": "plain read kernel (libawq_bench.so)", "bytes": n * 4, "us": round(read_us, 3),
                        "GB_per_s": round(n * 4 / read_us / 1e3, 1),
                        "frac": round(n * 4 / read_us / 1e3 / HBM_PEAK_GBS, 4)},
        "empty_launch": {"op": "kernel that does nothing, 448 work-groups of 256 threads (libawq_bench.so)",
                         "us": round(empty_us, 3)},
        "device_copy": {"op": "Tensor.copy_", "bytes_moved": 2 * n * 4, "us": round(copy_us, 3),
                        "GB_per_s": round(2 * n * 4 / copy_us / 1e3, 1),
                        "frac": round(2 * n * 4 / copy_us / 1e3 / HBM_PEAK_GBS, 4)},
        "vendor_fp16_linear_prefill_shape": {
            "op": "torch.nn.functional.linear, float16 weight (N, K), bias", "M": M, "K": K,
            "N": N, "us": round(lin_us, 3),
            "TFLOP_per_s": round(2 * M * N * K / lin_us / 1e6, 1),
            "frac": round(2 * M * N * K / lin_us / 1e6 / FP16_MFMA_PEAK_TFLOPS, 4)},
    }


def blas_thread_count():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def time_oracle(fn, budget_s):
    """Median wall time of fn() over repeated runs within about budget_s."""
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 20:
            break
    return statistics.median(times), len(times)


def cpu_baseline(p, g, budget_s, sample_rows=None):
    """The oracle, as it stands, on the host cores (rank 0 only)."""
    import oracle
    x = p["x"] if sample_rows is None else p["x"][:sample_rows]
    t, n = time_oracle(
        lambda: oracle.awq_linear_ref(x, p["qweight"], p["qzeros"], p["scales"], p["bias"], g),
        budget_s)
    return t, n, blas_thread_count()


def sweep_point(torch, awq, dev, name, M, g):
    """One workload point timed like the headline legs, printed as a JSON
    line against its binding roof; returns its time per call (ms) and
    whether it has a bias."""
    spec = dict(source=name, M=M, group_size=g)
    print(f"[sweep] {name} M={M} g={g}", file=sys.stderr, flush=True)
    r = run_leg(torch, awq, spec, None, 10, dev)
    sec = r["ms_per_step"] * 1e-3
    gbs = r["nbytes"] / sec / 1e9
    tfs = r["nflops"] / sec / 1e12
    # The binding roof: whichever takes longer at peak.
    hbm = r["nbytes"] / HBM_PEAK_GBS >= r["nflops"] / FP16_MFMA_PEAK_TFLOPS / 1e3
    print(json.dumps({
        "workload": name, "M": M, "K": r["K"], "N": r["N"], "group_size": g,
        "bias": r["p"]["bias"] is not None, "kernel": r["path"],
        "us_per_call": round(r["ms_per_step"] * 1e3, 3),
        "GB_per_s": round(gbs, 1), "TFLOP_per_s": round(tfs, 2),
        "bound": "hbm" if hbm else "mfma",
        "frac": round(gbs / HBM_PEAK_GBS if hbm else tfs / FP16_MFMA_PEAK_TFLOPS, 4),
        "bytes": r["nbytes"], "flops": r["nflops"], "copies_rotated": r["R"],
        "steps": r["steps"]}),
        flush=True)
    out = (r["ms_per_step"], r["K"], r["N"], r["p"]["bias"] is not None)
    del r
    torch.cuda.empty_cache()
    return out


def points(torch, awq, dev, specs):
    """The points named on the command line: WORKLOAD:M[,M...][:GROUP_SIZE]."""
    import awq_inputs
    for spec in specs:
        parts = spec.split(":")
        if len(parts) not in (2, 3) or parts[0] not in awq_inputs.WORKLOADS:
            raise SystemExit(f"--points: expected WORKLOAD:M[,M...][:GROUP_SIZE], got {spec!r}")
        g = int(parts[2]) if len(parts) == 3 else awq_inputs.WORKLOADS[parts[0]].group_sizes[0]
        for M in parts[1].split(","):
            sweep_point(torch, awq, dev, parts[0], int(M), g)


def sweep(torch, awq, dev):
    """Every point of every named workload, timed like the headline legs."""
    import awq_inputs
    fused = {}
    for name, w in awq_inputs.WORKLOADS.items():
        if name.startswith("tiny"):
            continue                    # launch-bound, a parity case only
        for g in w.group_sizes:
            for M in w.Ms:
                ms, K, N, has_bias = sweep_point(torch, awq, dev, name, M, g)
                if g == 128:
                    fused[(name, M, K, N, has_bias)] = ms
    # awq_dequant on its own (HBM-bound: packed words, zeros and scales in,
    # the float16 weight out), at the two large weight shapes (W = 117 MB,
    # written with ordinary stores) and at one whose W (470 MB) is larger
    # than the last-level cache (nontemporal stores).
    for (K, N) in ((8192, 7168), (14336, 4096), (8192, 28672)):
        print(f"[sweep] awq_dequant K={K} N={N}", file=sys.stderr, flush=True)
        d_us = dequant_time_us(torch, awq, K, N, dev)
        G = K // 128
        nbytes = K * N // 2 + G * N // 2 + G * N * 2 + K * N * 2
        print(json.dumps({
            "workload": f"awq_dequant_k{K}_n{N}_g128", "K": K, "N": N, "group_size": 128,
            "kernel": "dequant", "us_per_call": round(d_us, 3),
            "GB_per_s": round(nbytes / (d_us * 1e-6) / 1e9, 1), "bound": "hbm",
            "frac": round(nbytes / (d_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes": nbytes}),
            flush=True)
    # The unquantised float16 baseline at the single-token shapes the pages
    # name (FastLinear / FastLinearROCm: K = 8192, N = 1280 or 7168), timed
    # the same way; the W4A16 time at the same shape gives the speed-up.
    import awq_inputs
    for (K, N) in ((8192, 1280), (8192, 7168)):
        d_us = dense_time_us(torch, awq, 1, K, N, dev)
        name = "decode_k8192_n1280" if N == 1280 else "decode_sweep_k8192_n7168"
        r = run_leg(torch, awq, dict(source=name, M=1, group_size=128), None, 10, dev)
        w4_us = r["ms_per_step"] * 1e3
        nbytes = K * N * 2 + K * 2 + N * 2
        t_cpu, n_cpu = dense_oracle_time(K, N)
        print(json.dumps({
            "workload": f"dense_fp16_baseline_m1_k{K}_n{N}", "M": 1, "K": K, "N": N,
            "kernel": "dense_gemv", "us_per_call": round(d_us, 3),
            "GB_per_s": round(nbytes / (d_us * 1e-6) / 1e9, 1), "bound": "hbm",
            "frac": round(nbytes / (d_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes": nbytes,
            "w4a16_us_per_call": round(w4_us, 3), "w4a16_speedup": round(d_us / w4_us, 2),
            "cpu_baseline": {"value": round(nbytes / t_cpu / 1e9, 3), "unit": "GB/s",
                             "cores": blas_thread_count(), "kind": "oracle",
                             "sample": f"the same product through oracle.dense_linear_ref "
                                       f"(float64), median of {n_cpu} runs of {t_cpu:.3f} s"}}),
            flush=True)
    # Weights under a row-to-group map, rebuilt once as grouped weights:
    # activation order (whole groups) and an uneven map (32-row blocks,
    # padded); each step reorders x's columns and runs the grouped kernels.
    for name, M, kind in (("decode_sweep_k8192_n7168", 1, "act_order"),
                          ("decode_sweep_k8192_n7168", 16, "act_order"),
                          ("prefill_qkv_m2048_k4096_n12288", 2048, "act_order"),
                          ("decode_sweep_k8192_n7168", 1, "uneven"),
                          ("prefill_qkv_m2048_k4096_n12288", 2048, "uneven")):
        print(f"[sweep] {kind} map {name} M={M}", file=sys.stderr, flush=True)
        spec = dict(source=name, M=M, group_size=128, gidx=kind)
        r = run_leg(torch, awq, spec, None, 10, dev)
        sec = r["ms_per_step"] * 1e-3
        gbs = r["nbytes"] / sec / 1e9
        tfs = r["nflops"] / sec / 1e12
        hbm = r["nbytes"] / HBM_PEAK_GBS >= r["nflops"] / FP16_MFMA_PEAK_TFLOPS / 1e3
        plain = fused.get((name, M, r["K"], r["N"], r["p"]["bias"] is not None))
        t_cpu, n_cpu, rows = gidx_oracle_time(r["p"], min(M, 16))
        cpu = {"value": round(r["nbytes"] * rows / M / t_cpu / 1e9, 3), "unit": "GB/s",
               "cores": blas_thread_count(), "kind": "oracle",
               "sample": f"first {rows} of the {M} rows through oracle.awq_linear_gidx_ref "
                         f"(map lookup, float16 dequant, float64 matmul), median of {n_cpu} runs "
                         f"of {t_cpu:.2f} s; GB/s scaled to the rows computed"}
        print(json.dumps({
            "workload": f"{kind}_map_{name}", "M": M, "K": r["K"], "N": r["N"],
            "group_size": 128, "map": kind, "sorted_rows": r["sorted_rows"],
            "kernel": (f"{r['path']} (gathers x through the order itself)"
                       if r["path"] == "decode" and M <= 4 and r["N"] % 32 == 0
                       else f"x reorder pass + {r['path']}"),
            "us_per_call": round(sec * 1e6, 3),
            "GB_per_s": round(gbs, 1), "TFLOP_per_s": round(tfs, 2),
            "bound": "hbm" if hbm else "mfma",
            "frac": round(gbs / HBM_PEAK_GBS if hbm else tfs / FP16_MFMA_PEAK_TFLOPS, 4),
            "bytes": r["nbytes"], "copies_rotated": r["R"],
            "grouped_us_per_call": round(plain * 1e3, 3) if plain else None,
            "cpu_baseline": cpu}), flush=True)
        del r
        torch.cuda.empty_cache()
    # Context at the batches of 32 rows and more: torch's float16 linear (the
    # vendor GEMM library) on an unquantised weight of the same shape, and
    # the unfused route (awq_dequant into a float16 weight, then that GEMM).
    for (name, M, K, N, bias), ms in fused.items():
        if M < 32:
            continue
        print(f"[sweep] vendor float16 GEMM M={M} K={K} N={N}", file=sys.stderr, flush=True)
        lin_us, unfused_us = vendor_gemm_times_us(torch, awq, M, K, N, bias, dev)
        flops = 2 * M * N * K
        print(json.dumps({
            "workload": f"vendor_fp16_gemm_{name}", "M": M, "K": K, "N": N, "bias": bias,
            "kernel": "torch.nn.functional.linear (float16 weight (N, K))",
            "us_per_call": round(lin_us, 3), "TFLOP_per_s": round(flops / lin_us / 1e6, 2),
            "bound": "mfma", "frac": round(flops / lin_us / 1e6 / FP16_MFMA_PEAK_TFLOPS, 4),
            "unfused_dequant_then_gemm_us": round(unfused_us, 3),
            "w4a16_fused_us_per_call": round(ms * 1e3, 3)}), flush=True)


def dense_oracle_time(K, N):
    """Oracle time of the unquantised single-token product (float64)."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(K + N)
    x = rng.standard_normal((1, K)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    return time_oracle(lambda: oracle.dense_linear_ref(x, w, None), 3.0)


def gidx_oracle_time(p, rows):
    """Oracle time of the forward under p's row-to-group map on the first
    `rows` rows."""
    import oracle
    x = p["x"][:rows]
    run = lambda: oracle.awq_linear_gidx_ref(x, p["qweight"], p["qzeros"], p["scales"],  # noqa: E731
                                             p["g_idx"], p["bias"])
    run()   # the first run pays for page faults of its large temporaries
    t, n = time_oracle(run, 4.0)
    return t, n, rows


def vendor_gemm_times_us(torch, awq, M, K, N, bias, dev, calls=None):
    """Per-call times of torch's float16 linear on a random (N, K) weight,
    and of awq_dequant (g=128) followed by a float16 matmul, each captured in
    a graph and replayed like the headline legs."""
    if calls is None:
        calls = auto_steps(2 * N * K, 2 * M * N * K)
    gen = torch.Generator(device="cpu").manual_seed(M + K + N)
    x = torch.randn((M, K), generator=gen).to(torch.float16).to(dev)
    ws = [(torch.randn((N, K), generator=gen) * 0.02).to(torch.float16).to(dev) for _ in range(2)]
    b = (torch.randn((N,), generator=gen) * 0.1).to(torch.float16).to(dev) if bias else None
    G = K // 128
    qw = torch.randint(-2**31, 2**31 - 1, (K, N // 8), generator=gen, dtype=torch.int32).to(dev)
    qz = torch.randint(-2**31, 2**31 - 1, (G, N // 8), generator=gen, dtype=torch.int32).to(dev)
    sc = (torch.rand((G, N), generator=gen) * 0.009 + 0.001).to(torch.float16).to(dev)
    wkn = torch.empty((K, N), dtype=torch.float16, device=dev)

    def linear(i):
        return torch.nn.functional.linear(x, ws[i % 2], b)

    def unfused(i):
        awq.dequant(qw, qz, sc, 128, out=wkn)
        y = torch.matmul(x, wkn)
        return y + b if b is not None else y

    return graph_time_us(torch, linear, calls, dev), graph_time_us(torch, unfused, calls, dev)


def dequant_time_us(torch, awq, K, N, dev, calls=None):
    """awq_dequant per-call time, packed weights rotated through >= 512 MiB
    (each copy writes its own float16 output)."""
    import awq_inputs
    p = awq_inputs.make_inputs(1, K, N, 128, seed=K + N)
    nbytes = K * N // 2 + K * N * 2
    if calls is None:
        calls = auto_steps(nbytes, 0)
    R = max(2, -(-ROTATE_BYTES // nbytes))
    base = {k: torch.from_numpy(p[k]).to(dev) for k in ("qweight", "qzeros", "scales")}
    cps = [{k: v.clone() for k, v in base.items()} for _ in range(R)]
    outs = [torch.empty((K, N), dtype=torch.float16, device=dev) for _ in range(R)]
    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        for i in range(5):
            c = cps[i % R]
            awq.dequant(c["qweight"], c["qzeros"], c["scales"], 128, out=outs[i % R])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(calls):
            c = cps[i % R]
            awq.dequant(c["qweight"], c["qzeros"], c["scales"], 128, out=outs[i % R])
    graph.replay()
    torch.cuda.synchronize()
    ms, _ = settled_replay_ms(torch, graph, stream, calls)
    us = ms * 1e3 / calls
    del graph, cps, outs
    torch.cuda.empty_cache()
    return us


def dense_time_us(torch, awq, M, K, N, dev, calls=None):
    """awq_dense_gemv per-call time, weights rotated through >= 512 MiB."""
    gen = torch.Generator(device="cpu").manual_seed(K + N)
    nbytes = K * N * 2
    if calls is None:
        calls = auto_steps(nbytes, 0)
    R = max(2, -(-ROTATE_BYTES // nbytes))
    ws = [(torch.randn((N, K), generator=gen) * 0.02).to(torch.float16).to(dev) for _ in range(R)]
    x = torch.randn((M, K), generator=gen).to(torch.float16).to(dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        for i in range(10):
            awq.dense_gemv(x, ws[i % R], None, out=y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(calls):
            awq.dense_gemv(x, ws[i % R], None, out=y)
    graph.replay()
    torch.cuda.synchronize()
    ms, _ = settled_replay_ms(torch, graph, stream, calls)
    return ms * 1e3 / calls


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--legs", default="decode,prefill",
                    help="comma-separated: decode, prefill, and refs (the same-box references "
                         "even with --no-configs)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config points and the same-box references")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (for profiler runs)")
    ap.add_argument("--points", nargs="+", metavar="WORKLOAD:M[,M...][:G]",
                    help="instead of the headline line, time only these workload points "
                         "(one JSON line each, like --sweep)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line, print one JSON line per point of "
                         "every named workload (all batch sizes and group sizes), each "
                         "against its binding roof: whichever of HBM bytes and MFMA flops "
                         "takes longer at peak")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the multi-GPU (sharded) path is not part of "
              "this build; rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_weight_quantized_awq_amd as awq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    awq.lib()
    if args.sweep:
        sweep(torch, awq, dev)
        return
    if args.points:
        points(torch, awq, dev, args.points)
        return
    legs = args.legs.split(",")
    res = {}
    for name, spec in (("decode", DECODE), ("prefill", PREFILL)):
        if name in legs:
            print(f"[bench] {name} leg: {spec['workload']}", file=sys.stderr, flush=True)
            res[name] = run_leg(torch, awq, spec, args.steps, args.warmup, dev)

    def decode_fields(r):
        gbs = r["nbytes"] / (r["ms_per_step"] * 1e-3) / 1e9
        return gbs, gbs

    out = {
        "metric": "W4A16 GEMM: decode GB/s (% HBM peak) at M=1; prefill TFLOP/s (% MFMA peak)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
    }
    if "decode" in res:
        r = res["decode"]
        gbs, kgbs = decode_fields(r)
        out.update({
            "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": r["ms_per_step"],
            "config": {"workload": DECODE["workload"], "M": r["M"], "K": r["K"], "N": r["N"],
                       "group_size": r["g"], "bias": False, "kernel": r["path"],
                       "weight_copies_rotated": r["R"], "bytes_per_step": r["nbytes"],
                       "hbm_peak_frac_whole_job": round(gbs / HBM_PEAK_GBS, 4),
                       "eager_ms_per_step": r["eager_ms"]},
            "roofline": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode"),
                         "graph_step_us": round(r["ms_per_step"] * 1e3, 3),
                         "single_launch_event_us": round(r["kern_avg_ms"] * 1e3, 3),
                         "untimed_settle_ms": round(r["settle_ms"], 1)},
        })
    if "prefill" in res:
        r = res["prefill"]
        tf = r["nflops"] / (r["ms_per_step"] * 1e-3) / 1e12
        ktf = tf
        pre = {"workload": PREFILL["workload"], "value": round(tf, 1), "unit": "TFLOP/s",
               "ms_per_step": r["ms_per_step"], "kernel": r["path"],
               "M": r["M"], "K": r["K"], "N": r["N"], "group_size": r["g"], "bias": True,
               "roofline": {"bound": "mfma", "achieved": round(ktf, 1),
                            "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(ktf / FP16_MFMA_PEAK_TFLOPS, 4),
                            "traffic": measured_traffic("prefill"),
                            "graph_step_us": round(r["ms_per_step"] * 1e3, 3),
                            "single_launch_event_us": round(r["kern_avg_ms"] * 1e3, 3),
                            "untimed_settle_ms": round(r["settle_ms"], 1)}}
        if "decode" not in res:
            out.update({"value": pre["value"], "unit": "TFLOP/s",
                        "ms_per_step": pre["ms_per_step"],
                        "config": {"workload": pre["workload"]}, "roofline": pre["roofline"]})
        out["prefill"] = pre

    if not args.no_configs:
        out["configs"] = config_points(torch, awq, dev)
    if not args.no_configs or "refs" in legs:
        print("[bench] same-box references", file=sys.stderr, flush=True)
        out["references"] = same_box_references(
            torch, dev, res["decode"]["nbytes"] if "decode" in res else 30537728)
    if not args.no_cpu_baseline and "decode" in res:
        r = res["decode"]
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        t, n, cores = cpu_baseline(r["p"], r["g"], budget_s=12.0)
        out["cpu_baseline"] = {
            "value": round(r["nbytes"] / t / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"the full decode problem (M=1, K=8192, N=7168, g=128) through the "
                      f"numpy oracle (unpack, float16 dequant, float64 matmul), median of {n} "
                      f"runs of {t:.2f} s; elementwise steps single-threaded, BLAS on "
                      f"{cores} threads"}
    if not args.no_cpu_baseline and "prefill" in res:
        r = res["prefill"]
        rows = 128
        t, n, cores = cpu_baseline(r["p"], r["g"], budget_s=12.0, sample_rows=rows)
        out["prefill"]["cpu_baseline"] = {
            "value": round(2 * rows * r["K"] * r["N"] / t / 1e12, 5), "unit": "TFLOP/s",
            "cores": cores, "kind": "oracle",
            "sample": f"first {rows} of the 2048 rows of the prefill problem through the numpy "
                      f"oracle (full dequant + float64 matmul), median of {n} runs of {t:.2f} s"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
