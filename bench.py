#!/usr/bin/env python3
"""Benchmark of the ternary-g128 decode hot path on one MI355X.

One step = the rotated decode path for one token: sign flip + signed
normalized Walsh-Hadamard transform (block 4096) of a bfloat16 activation
row, then the ternary-g128 GEMV M=1, K=4096 -> N=12288 on the rotated
binary32 activations.  Inputs are seeded synthetic arrays resident in HBM
before timing starts.  Weights rotate over a pool of distinct copies larger
than 1 GiB so that neither L2 nor the 256 MB MALL can serve repeats, and the
K timed steps are captured in one HIP graph (host launch overhead would
otherwise dominate microsecond kernels).

Prints one JSON line.  `value` is algorithmic bytes per step / step time.
`roofline` covers the dominant kernel (the GEMV), timed with HIP events on
the stream it runs on.  `cpu_baseline` is the FP64 oracle on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
POOL_BYTES = 1 << 30           # rotate weights over at least this much HBM
METRIC = "ternary GEMV HBM GB/s (M=1) & % of peak; pp512 GEMM TFLOP/s & % MFMA peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--reps", type=int, default=7,
                   help="timed replays of the headline graph (each after a cache flush)")
    p.add_argument("--workload", default="rotated",
                   choices=["rotated", "sweep", "prefill", "chain", "base3", "binary", "tiny", "floor", "copy"],
                   help="rotated: the headline step; sweep / prefill / chain / base3 / binary / tiny: extra "
                        "measurements; floor: load-only kernels over the decode byte counts; "
                        "copy: a plain device copy of known size (counter calibration)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-secondary", action="store_true", help="headline line only")
    p.add_argument("--no-clocks", action="store_true",
                   help="skip reading the clocks under load (1.5 s of replays; for profiled runs)")
    return p.parse_args()


def gemv_bytes(M, K, N, x_bytes):
    return N * K // 4 + 2 * N * K // 128 + M * K * x_bytes + M * N * 4


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_rotated_M1_K4096_N12288_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "ternary_weight_g128_amd", "csrc", f)
                  for f in ("tern_kernels.hip", "tern_device.h", "tern_h64.h")]


def measured_traffic():
    """HBM bytes per launch of the fused kernel from the committed counter
    summary, or None when the kernel source changed since it was taken."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    src = h.hexdigest()
    if fields.get("kernel_source_sha256") != src:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def bench_copy(torch, nbytes=256 << 20, reps=5):
    """A plain device-to-device copy of nbytes (reads nbytes, writes nbytes):
    the reference for scaling FETCH_SIZE / WRITE_SIZE counters to bytes."""
    src = torch.randn(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}


def rotated_step_bytes(w):
    """Algorithmic HBM bytes of one rotated decode step: packed codes, FP16
    scales, the bfloat16 activation row, the int8 signs and the FP32 output."""
    return (w.N * w.K // 4 + 2 * w.N * w.K // 128 + w.M * w.K * 2 + w.K + w.M * w.N * 4)


def make_pool(tern, torch, t, s, nbytes_each):
    codes, s2 = tern.tern_pack(t, s)
    c0, s0 = tern.to_device(codes, s2)
    copies = max(2, -(-POOL_BYTES // nbytes_each))
    pool = [(c0, s0)] + [(c0.clone(), s0.clone()) for _ in range(copies - 1)]
    torch.cuda.synchronize()
    return pool


class Flusher:
    """Evicts L2 and the 256 MB MALL between timed replays by reading a
    1 GiB buffer (a torch reduction on the current stream).  It only reads,
    so no dirty lines are left for the timed replay to write back."""

    def __init__(self, torch, nbytes=1 << 30):
        self.buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")

    def __call__(self):
        self.buf.sum()


_FLUSH = None


def flusher(torch):
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = Flusher(torch)
    return _FLUSH


def capture(torch, fn, steps):
    """Capture `steps` calls fn(0) .. fn(steps - 1) in one HIP graph."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    return g


def time_graph(torch, fn, steps, reps=3):
    """Capture `steps` calls of fn(i) in one HIP graph and replay it `reps`
    times, timing each replay with HIP events on the replay stream.  One
    untimed replay uploads the graph first; before every timed replay the
    flusher streams 1 GiB through L2 and the MALL, so no timed replay finds
    the weights it reads in a cache (whatever the step count).  The flush,
    the start event, the replay and the end event are queued together
    (the flush keeps the GPU busy while the host submits the replay), so the
    interval between the events is the GPU time of the steps alone, not the
    host's submission of the graph.  Returns the median replay time in ms,
    the graph, and median / p10 / p90."""
    g = capture(torch, fn, steps)
    g.replay()                       # upload / first replay, untimed
    torch.cuda.synchronize()
    fl = flusher(torch)
    cur = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        fl()
        start.record(cur)
        g.replay()
        end.record(cur)
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end))
    t = np.array(times)
    stats = {"replays": reps, "steps_per_replay": steps,
             "median_ms": float(np.median(t)), "p10_ms": float(np.percentile(t, 10)),
             "p90_ms": float(np.percentile(t, 90))}
    return stats["median_ms"], g, stats


def per_step_us(stats):
    """Median / p10 / p90 of the per-step time (us) over timed replays."""
    n = stats["steps_per_replay"]
    return {"median_us": 1e3 * stats["median_ms"] / n, "p10_us": 1e3 * stats["p10_ms"] / n,
            "p90_us": 1e3 * stats["p90_ms"] / n, "replays": stats["replays"], "steps_per_replay": n}


def _gpu_sysfs_dir(torch):
    """The sysfs directory of device 0 (its PCI address from the device
    properties), or the only DRM card with clock tables; None if neither."""
    import glob
    p = torch.cuda.get_device_properties(0)
    bus = getattr(p, "pci_bus_id", None)
    if bus is not None:
        d = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (getattr(p, "pci_domain_id", 0) or 0, bus,
                                                      getattr(p, "pci_device_id", 0) or 0)
        if os.path.exists(os.path.join(d, "pp_dpm_sclk")):
            return d
    cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    return os.path.dirname(cards[0]) if len(cards) == 1 else None


def _dpm_level(path):
    """The current level of a pp_dpm_* table (the line marked '*')."""
    try:
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return line.split(":", 1)[1].replace("*", "").strip()
    except OSError:
        return None
    return None


def clocks_under_load(torch, g, replay_ms, seconds=1.5):
    """GPU clocks read from the device's sysfs clock tables while the timed
    graph replays back to back (about `seconds` of queued GPU work), so the
    clocks are the ones the kernels run at (no helper process is started).
    Returns the current sclk / mclk levels (or the reason they are missing)."""
    n = int(max(1, seconds * 1e3 / max(replay_ms, 1e-3)))
    n = min(n, 20000)
    d = _gpu_sysfs_dir(torch)
    for _ in range(n):
        g.replay()
    res = {}
    if d is not None:
        for key in ("sclk", "mclk", "fclk", "socclk"):
            v = _dpm_level(os.path.join(d, "pp_dpm_" + key))
            if v is not None:
                res[key] = v
    torch.cuda.synchronize()
    if not res:
        res["error"] = "no readable clock table for device 0"
    res["replays_queued"] = n
    return res


def rotated_step_setup(tern, torch, synth):
    w = synth.ROTATED
    seed = 11
    t = synth.ternary(seed, w.N, w.K, w.p_zero)
    s = synth.scales_f16(seed, w.N, w.K)
    x = synth.activations_bf16(seed, w.M, w.K)
    d = synth.signs(seed, w.K)
    wbytes = tern.tern_codes_bytes(w.N, w.K) + tern.tern_scales_bytes(w.N, w.K)
    pool = make_pool(tern, torch, t, s, wbytes)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    dd = torch.from_numpy(d).cuda()
    xr = torch.empty((w.M, w.K), dtype=torch.float32, device="cuda")
    y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    return w, (t, s, x, d), pool, xd, dd, xr, y


def bench_rotated(args, tern, torch, synth):
    w, host, pool, xd, dd, xr, y = rotated_step_setup(tern, torch, synth)
    P = len(pool)

    # one step = sign flip + rotation + GEMV, fused in one kernel launch
    def step(i):
        c, s = pool[i % P]
        tern.tern_rotate_gemv(xd, dd, w.rotate_block, c, s, out=y)

    # the same path as two launches (transform, then GEMV), for reference
    def two_launch_step(i):
        c, s = pool[i % P]
        tern.tern_fwht(xd, dd, w.rotate_block, out=xr)
        tern.tern_gemv(xr, c, s, out=y)

    def gemv_only(i):
        c, s = pool[i % P]
        tern.tern_gemv(xr, c, s, out=y)

    def fwht_only(i):
        tern.tern_fwht(xd, dd, w.rotate_block, out=xr)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the timed region: exactly `steps` steps per replay, synchronized on
    # both sides; the median over `reps` replays (each after a cache flush)
    torch.cuda.synchronize()
    step_ms, g, stats = time_graph(torch, step, args.steps, reps=args.reps)
    ms_per_step = step_ms / args.steps
    two_ms, _, _ = time_graph(torch, two_launch_step, args.steps)
    gemv_ms, _, _ = time_graph(torch, gemv_only, args.steps)
    fwht_ms, _, _ = time_graph(torch, fwht_only, args.steps)
    kernel_us = 1e3 * ms_per_step   # the step is one kernel
    gemv_us = 1e3 * gemv_ms / args.steps
    fwht_us = 1e3 * fwht_ms / args.steps
    clocks = None if args.no_clocks else clocks_under_load(torch, g, step_ms)

    # sanity: a replay of the timed graph reproduces the eager result
    step(args.steps - 1)
    torch.cuda.synchronize()
    y_eager = y.clone()
    y.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y, y_eager), "graph replay differs from eager execution"

    # algorithmic bytes of the fused step: codes + scales + bf16 x + signs + y
    step_bytes = rotated_step_bytes(w)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = step_bytes / (kernel_us * 1e-6) / 1e9
    res = {
        "value": value,
        "ms_per_step": ms_per_step,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic()},
        "detail": {"kernel": "gemv_kernel<2, true, TPW, true, 1> (fused rotation + GEMV)",
                   "kernel_us": kernel_us, "step_bytes": step_bytes,
                   "step_us_over_replays": per_step_us(stats), "clocks_under_load": clocks,
                   "two_launch_step_us": 1e3 * two_ms / args.steps,
                   "gemv_only_us": gemv_us, "gemv_only_GBps": gemv_bytes(w.M, w.K, w.N, 4) / (gemv_us * 1e-6) / 1e9,
                   "fwht_only_us": fwht_us,
                   "pool_copies": P, "pool_bytes": P * (tern.tern_codes_bytes(w.N, w.K) +
                                                        tern.tern_scales_bytes(w.N, w.K))},
    }
    return w, host, res


def host_cpu():
    """Host CPU model name and the cores this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


def _time_oracle_steps(w, host, threads, min_seconds):
    import oracle
    t, s, x, d = host
    codes = oracle.encode(t)
    x64 = oracle.bf16_bits_to_f64(x)
    reps = 0
    t0 = time.perf_counter()
    while True:
        xr = oracle.fwht(x64, d, w.rotate_block)
        oracle.matmul(xr, codes, s, w.K, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return reps, el


def cpu_baseline(w, host, seconds_all=10.0, seconds_one=8.0):
    """The FP64 oracle, as it stands, on the same step: explicit-matrix
    rotation, then the naive matmul over all rows.  The reported value uses
    every host core (the matmul's outputs shared over threads, each output
    the same k-ordered sum; the small rotation stays on one thread); the
    single-thread rate of the same program is reported beside it."""
    import oracle
    model, cores = host_cpu()
    threads = max(1, min(cores, oracle.max_threads()))
    step_bytes = rotated_step_bytes(w)
    reps, el = _time_oracle_steps(w, host, threads, seconds_all)
    reps1, el1 = _time_oracle_steps(w, host, 1, seconds_one)
    return {"value": step_bytes * reps / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "host_cores": cores,
            "single_core_value": step_bytes * reps1 / el1 / 1e9,
            "sample": f"{reps} full rotated decode steps in {el:.1f} s on {threads} threads "
                      f"({reps1} in {el1:.1f} s on 1 thread): FP64 explicit-Hadamard rotation "
                      f"+ naive FP64 matmul over all {w.N} rows"}


def cpu_secondary(synth, seconds=2.0):
    """The FP64 oracle on bounded samples of the prefill GEMM, the decode GEMV
    shapes and every link shape of the 27B-class decode pass: a slice of
    output rows over the full K and all M rows of x, on every host core
    (outputs shared over threads).  Rates are per output computed, so they
    compare with the GPU figures of the same shapes; the pass's tokens/s is
    extrapolated from the per-row times of its link shapes, and labelled so."""
    import oracle
    model, cores = host_cpu()
    threads = max(1, min(cores, oracle.max_threads()))
    out = {}

    def rate(M, K, rows, p0, outl, seed):
        t = synth.ternary(seed, rows, K, p0)
        s = synth.scales_f16(seed, rows, K)
        x = synth.activations_bf16(seed, M, K, outl)
        codes = oracle.encode(t)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.matmul(x, codes, s, K, threads=threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        return reps, el

    cases = [("prefill", w.M, w.K, w.N, w.p_zero, w.outlier_frac) for w in synth.PREFILL] + \
            [("decode", 1, 5120, 17408, 1 / 3, 0.0), ("decode", 1, 17408, 5120, 1 / 3, 0.0)]
    for kind, M, K, N, p0, outl in cases:
        rows = threads if kind == "prefill" else 16 * threads
        reps, el = rate(M, K, rows, p0, outl, 31 + K)
        flops = 2.0 * M * rows * K * reps
        byts = (rows * K // 4 + 2 * rows * K // 128 + M * K * 2 + M * rows * 4) * reps
        out[f"{kind}_M{M}_K{K}_N{N}"] = {
            "GFLOP/s": flops / el / 1e9, "GB/s": byts / el / 1e9, "cores": threads, "kind": "oracle",
            "sample": f"{reps} x ({rows} of {N} output rows, M={M}, full K={K}), {el:.1f} s"}
    # the 27B-class pass: seconds per output row of each distinct link shape
    links = synth.chain_links()
    shapes = sorted(set(links))
    per_row = {}
    for (K, N) in shapes:
        rows = 16 * threads
        reps, el = rate(1, K, rows, 1 / 3, 0.0, 53 + K + N)
        per_row[(K, N)] = el / (reps * rows)
    pass_s = sum(per_row[(K, N)] * N for (K, N) in links)
    packed = sum(N * K // 4 + 2 * N * K // 128 for (K, N) in links)
    out["decode_pass_27b_class"] = {
        "tokens_per_s": 1.0 / pass_s, "s_per_pass": pass_s, "GB/s": packed / pass_s / 1e9,
        "cores": threads, "kind": "oracle", "cpu_model": model,
        "sample": f"extrapolated: {len(shapes)} link shapes timed on {16 * threads}-row slices "
                  f"(about {seconds:.0f} s each), scaled to the {len(links)} links' full row counts"}
    return out


def bench_tiny(tern, torch, synth, steps):
    """The tiny GEMV (M=1, K=1024, N=1024, binary32 x): the latency of one
    call with its 0.28 MB of weights resident in L2 (the same weights every
    step), and, labelled as such, the rate over a rotated pool of copies."""
    w = synth.TINY
    seed = 41
    t = synth.ternary(seed, w.N, w.K)
    s = synth.scales_f16(seed, w.N, w.K)
    x = torch.from_numpy(synth.activations_f32(seed, w.M, w.K)).cuda()
    y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    pool = make_pool(tern, torch, t, s, tern.tern_codes_bytes(w.N, w.K) + tern.tern_scales_bytes(w.N, w.K))
    P = len(pool)

    def same(i):
        tern.tern_gemv(x, *pool[0], out=y)

    def rotated(i):
        tern.tern_gemv(x, *pool[i % P], out=y)

    for i in range(5):
        same(i)
    ms_same, _, st_same = time_graph(torch, same, steps)
    ms_rot, _, _ = time_graph(torch, rotated, steps)
    us_rot = 1e3 * ms_rot / steps
    byts = gemv_bytes(w.M, w.K, w.N, 4)
    return {"latency_us_weights_in_l2": per_step_us(st_same),
            "rotated_pool_us": us_rot, "rotated_pool_GB/s": byts / (us_rot * 1e-6) / 1e9,
            "bytes": byts, "pool_copies": P}


def bench_floor(tern, torch, synth, steps):
    """Load-only floor: a kernel that only reads (16-byte loads, several in
    flight per thread, one store per workgroup) exactly the packed-weight
    bytes of each decode GEMV shape, launched once per step from a graph over
    a rotated pool like the GEMV itself.  The best of a few launch shapes is
    reported: no GEMV over the same bytes, launched once per call, can beat
    it."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "ternary_weight_g128_amd", "libtern_bench.so"))
    lib.tern_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.tern_bench_read.restype = ctypes.c_int
    sink = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    out = {}
    for (M, K, N) in ((1, 4096, 12288), (1, 5120, 17408), (1, 17408, 5120)):
        nbytes = N * K // 4 + 2 * N * K // 128
        nbytes = (nbytes + 15) // 16 * 16
        copies = max(2, -(-POOL_BYTES // nbytes))
        pool = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i & 0xff) for i in range(copies)]
        best = None
        for wgs in (256, 512, 768, 1024, 2048):
            for depth in (1, 2, 4, 8):
                def fn(i, wgs=wgs, depth=depth):
                    rc = lib.tern_bench_read(ctypes.c_void_p(pool[i % copies].data_ptr()), nbytes, wgs, depth,
                                             ctypes.c_void_p(sink.data_ptr()),
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                    assert rc == 0, rc
                fn(0)
                ms, _, _ = time_graph(torch, fn, steps, reps=2)
                us = 1e3 * ms / steps
                if best is None or us < best[0]:
                    best = (us, wgs, depth)
        us, wgs, depth = best
        out[f"read_K{K}_N{N}"] = {"bytes": nbytes, "us": us, "GB/s": nbytes / (us * 1e-6) / 1e9,
                                  "frac_hbm": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                  "workgroups": wgs, "loads_in_flight_per_thread": depth}
        del pool
        torch.cuda.empty_cache()
    return out


def bench_sweep(tern, torch, synth, steps):
    """Decode GEMV at M = 1, 16 on both MLP shapes, rotated pool, graph-timed."""
    out = {}
    for (K, N) in ((5120, 17408), (17408, 5120)):
        seed = 5 + K
        t = synth.ternary(seed, N, K)
        s = synth.scales_f16(seed, N, K)
        pool = make_pool(tern, torch, t, s, tern.tern_codes_bytes(N, K) + tern.tern_scales_bytes(N, K))
        P = len(pool)
        for M in (1, 2, 4, 8, 16):
            x = synth.activations_bf16(seed, M, K)
            xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
            y = torch.empty((M, N), dtype=torch.float32, device="cuda")

            def fn(i, xd=xd, y=y):
                c, s_ = pool[i % P]
                tern.tern_gemv(xd, c, s_, out=y)

            for i in range(5):
                fn(i)
            ms, _, _ = time_graph(torch, fn, steps)
            us = 1e3 * ms / steps
            gbs = gemv_bytes(M, K, N, 2) / (us * 1e-6) / 1e9
            out[f"M{M}_K{K}_N{N}"] = {"us": us, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}
        del pool
        torch.cuda.empty_cache()
    return out


def t5_gemv_bytes(M, K, N):
    """Algorithmic bytes of a GEMV over the base-3 layout: ceil(K/640) * 128
    bytes per row, FP16 scales, bf16 activations, fp32 output."""
    return N * ((K // 128 + 4) // 5) * 128 + 2 * N * K // 128 + M * K * 2 + M * N * 4


def bench_t5(tern, torch, synth, steps):
    """Decode GEMV over the base-3 layout (1.6 bits/weight) beside the 2-bit
    GEMV on the same weights, M = 1 and 16, rotated pools, graph-timed."""
    out = {}
    for (K, N) in ((4096, 12288), (5120, 17408), (17408, 5120)):
        seed = 7 + K
        t = synth.ternary(seed, N, K)
        s = synth.scales_f16(seed, N, K)
        codes, s2 = tern.tern_pack(t, s)
        data = tern.tern_pack_t5(codes, K)
        d0 = torch.from_numpy(data).cuda()
        s0 = torch.from_numpy(s2.view(np.int16)).cuda()
        copies = max(2, -(-POOL_BYTES // (data.size + s2.nbytes)))
        pool = [(d0, s0)] + [(d0.clone(), s0.clone()) for _ in range(copies - 1)]
        pool2 = make_pool(tern, torch, t, s, tern.tern_codes_bytes(N, K) + tern.tern_scales_bytes(N, K))
        for M in (1, 16):
            x = synth.activations_bf16(seed, M, K)
            xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
            y = torch.empty((M, N), dtype=torch.float32, device="cuda")

            def fn(i, xd=xd, y=y):
                d, s_ = pool[i % len(pool)]
                tern.tern_gemv_t5(xd, d, s_, out=y)

            def fn2(i, xd=xd, y=y):
                c, s_ = pool2[i % len(pool2)]
                tern.tern_gemv(xd, c, s_, out=y)

            for i in range(5):
                fn(i)
                fn2(i)
            ms, _, _ = time_graph(torch, fn, steps)
            ms2, _, _ = time_graph(torch, fn2, steps)
            us, us2 = 1e3 * ms / steps, 1e3 * ms2 / steps
            gbs = t5_gemv_bytes(M, K, N) / (us * 1e-6) / 1e9
            out[f"M{M}_K{K}_N{N}"] = {"us": us, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                                      "bytes": t5_gemv_bytes(M, K, N), "us_2bit": us2,
                                      "bytes_2bit": gemv_bytes(M, K, N, 2)}
        del pool, pool2, d0, s0
        torch.cuda.empty_cache()
    return out


def b1_gemv_bytes(M, K, N):
    """Algorithmic bytes of a GEMV over the binary variant: K/8 bytes of sign
    bits per row, FP16 scales, bf16 activations, fp32 output."""
    return N * K // 8 + 2 * N * K // 128 + M * K * 2 + M * N * 4


def bench_b1(tern, torch, synth, steps):
    """Decode GEMV over the binary variant (1.125 bits/weight) beside the
    2-bit GEMV on the same +-1 weights (their ternary codes), M = 1 and 4,
    rotated pools, graph-timed."""
    out = {}
    for (K, N) in ((5120, 17408), (17408, 5120)):
        seed = 11 + K
        b = synth.ternary(seed, N, K, 0.0)
        s = synth.scales_f16(seed, N, K)
        bits = tern.tern_pack_b1(b)
        b0 = torch.from_numpy(bits.view(np.int32)).cuda()
        s0 = torch.from_numpy(s.view(np.int16)).cuda()
        copies = max(2, -(-POOL_BYTES // (bits.nbytes + s.nbytes)))
        pool = [(b0, s0)] + [(b0.clone(), s0.clone()) for _ in range(copies - 1)]
        pool2 = make_pool(tern, torch, b, s, tern.tern_codes_bytes(N, K) + tern.tern_scales_bytes(N, K))
        for M in (1, 4):
            x = synth.activations_bf16(seed, M, K)
            xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
            y = torch.empty((M, N), dtype=torch.float32, device="cuda")

            def fn(i, xd=xd, y=y):
                w, s_ = pool[i % len(pool)]
                tern.tern_gemv_b1(xd, w, s_, out=y)

            def fn2(i, xd=xd, y=y):
                c, s_ = pool2[i % len(pool2)]
                tern.tern_gemv(xd, c, s_, out=y)

            for i in range(5):
                fn(i)
                fn2(i)
            ms, _, _ = time_graph(torch, fn, steps)
            ms2, _, _ = time_graph(torch, fn2, steps)
            us, us2 = 1e3 * ms / steps, 1e3 * ms2 / steps
            gbs = b1_gemv_bytes(M, K, N) / (us * 1e-6) / 1e9
            out[f"M{M}_K{K}_N{N}"] = {"us": us, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                                      "bytes": b1_gemv_bytes(M, K, N), "us_2bit": us2,
                                      "bytes_2bit": gemv_bytes(M, K, N, 2)}
        del pool, pool2, b0, s0
        torch.cuda.empty_cache()
    return out


def bench_prefill(tern, torch, synth, steps):
    out = {}
    for w in synth.PREFILL:
        seed = 9 + w.K
        t = synth.ternary(seed, w.N, w.K, w.p_zero)
        s = synth.scales_f16(seed, w.N, w.K)
        codes, s2 = tern.tern_pack(t, s)
        c, sd = tern.to_device(codes, s2)
        x = synth.activations_bf16(seed, w.M, w.K, w.outlier_frac)
        xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
        y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        ws_n = tern.tern_gemm_workspace_bytes(w.M, w.N, w.K)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

        def fn(i):
            tern.tern_gemm(xd, c, sd, out=y, workspace=ws)

        for i in range(3):
            fn(i)
        ms, _, _ = time_graph(torch, fn, steps)
        us = 1e3 * ms / steps
        tf = 2.0 * w.M * w.N * w.K / (us * 1e-6) / 1e12
        out[f"M{w.M}_K{w.K}_N{w.N}"] = {"us": us, "TFLOP/s": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS}
    return out


def bench_chain(tern, torch, synth, passes=5):
    """The 27B-class decode weight pass: 64 blocks of four chained GEMVs
    (gate and up as one matrix of both, since they take the same input) plus
    the LM head (257 dependent launches), M=1, bf16 activations.  Where the
    lengths match, a link's output (bf16) is the next link's input (the down
    projection takes the up half of the gate/up output); the 6144-wide input
    of each block's second link is a fixed seeded vector.
    Weights are drawn and packed on the GPU (6.49 GB resident).  `passes`
    full passes are captured in one HIP graph and timed, and timed again as
    plain launches on the stream."""
    gen = synth.device_generator(20)
    links = synth.chain_links()
    weights = []
    for (K, N) in links:
        codes = torch.empty((N, K // 16), dtype=torch.int32, device="cuda")
        rows = max(1, (64 << 20) // K)
        for n0 in range(0, N, rows):
            nr = min(rows, N - n0)
            tern.tern_pack_device(synth.device_ternary(gen, nr, K), out=codes[n0:n0 + nr])
        s = synth.device_scales_f16(gen, N, K).view(torch.int16)
        weights.append((codes, s))
    x5120 = synth.device_activations_bf16(gen, 1, 5120)
    x6144 = synth.device_activations_bf16(gen, 1, 6144)
    cur = torch.empty((1, 5120), dtype=torch.bfloat16, device="cuda")
    h5120 = torch.empty((1, 5120), dtype=torch.bfloat16, device="cuda")
    qkv = torch.empty((1, 12288), dtype=torch.bfloat16, device="cuda")
    gate_up = torch.empty((1, 2 * synth.CHAIN_GATE_UP), dtype=torch.bfloat16, device="cuda")
    up = gate_up[:, synth.CHAIN_GATE_UP:]
    logits = torch.empty((1, synth.LM_HEAD[1]), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def one_pass(_i):
        cur.copy_(x5120)
        nl = len(synth.CHAIN_BLOCK)
        for b in range(synth.CHAIN_BLOCKS):
            w = weights[nl * b: nl * b + nl]
            tern.tern_gemv(cur, *w[0], out=qkv)           # 5120 -> 12288
            tern.tern_gemv(x6144, *w[1], out=h5120)       # 6144 -> 5120 (fixed input)
            tern.tern_gemv(h5120, *w[2], out=gate_up)     # 5120 -> 17408 + 17408
            tern.tern_gemv(up, *w[3], out=cur)            # 17408 -> 5120
        tern.tern_gemv(cur, *weights[-1], out=logits)     # LM head

    one_pass(0)
    torch.cuda.synchronize()
    ms, _, _ = time_graph(torch, one_pass, passes)
    ms_pass = ms / passes
    # the same passes as plain back-to-back launches on the stream (host
    # launch cost included), HIP events around them
    cur_stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(cur_stream)
    for i in range(passes):
        one_pass(i)
    end.record(cur_stream)
    torch.cuda.synchronize()
    ms_eager = start.elapsed_time(end) / passes
    packed = sum(tern.tern_codes_bytes(N, K) + tern.tern_scales_bytes(N, K) for (K, N) in links)
    act = sum(2 * K + (4 if i == len(links) - 1 else 2) * N for i, (K, N) in enumerate(links))
    return {"gemvs": len(links), "packed_bytes": packed, "activation_bytes": act,
            "ms_per_pass": ms_pass, "tokens_per_s": 1e3 / ms_pass,
            "GB/s": (packed + act) / (ms_pass * 1e-3) / 1e9,
            "frac_hbm": (packed + act) / (ms_pass * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "ms_per_pass_eager": ms_eager, "tokens_per_s_eager": 1e3 / ms_eager}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; the kernels are single-GPU "
                                   "and --gpus above 1 is not supported", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import synth
    import ternary_weight_g128_amd as tern
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.workload == "copy":
        print(json.dumps({"copy": bench_copy(torch)}))
        return
    if args.workload in ("sweep", "prefill", "tiny", "floor"):
        fn = {"sweep": bench_sweep, "prefill": bench_prefill, "tiny": bench_tiny, "floor": bench_floor}
        print(json.dumps({args.workload: fn[args.workload](tern, torch, synth, args.steps)}))
        return
    if args.workload == "chain":
        print(json.dumps({"chain": bench_chain(tern, torch, synth)}))
        return
    if args.workload == "base3":
        print(json.dumps({"base3": bench_t5(tern, torch, synth, args.steps)}))
        return
    if args.workload == "binary":
        print(json.dumps({"binary": bench_b1(tern, torch, synth, args.steps)}))
        return

    w, host, res = bench_rotated(args, tern, torch, synth)
    line = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "rotated decode: sign flip + normalized Walsh-Hadamard (block 4096) "
                               "+ ternary-g128 GEMV M=1 K=4096 N=12288",
                   "M": w.M, "K": w.K, "N": w.N, "graph_captured": True,
                   "weight_pool_bytes": res["detail"]["pool_bytes"]},
        "roofline": res["roofline"],
        "detail": res["detail"],
    }
    if not args.no_secondary:
        line["secondary"] = {
            "tiny_gemv_latency": bench_tiny(tern, torch, synth, 200),
            "load_only_floor": bench_floor(tern, torch, synth, 200),
            "decode_sweep_gemv": bench_sweep(tern, torch, synth, 200),
            "prefill_gemm": bench_prefill(tern, torch, synth, 20),
            "decode_pass_27b_class": bench_chain(tern, torch, synth),
            "decode_gemv_base3": bench_t5(tern, torch, synth, 200),
            "decode_gemv_binary": bench_b1(tern, torch, synth, 200),
        }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, host)
        if not args.no_secondary:
            line["secondary"]["cpu_oracle"] = cpu_secondary(synth)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
