#!/usr/bin/env python3
"""Benchmark of the attention forward on one MI355X.

A step is one fa_fwd call over the headline workload: one bf16 head, N = 8192,
d = dv = 128, causal (the single-head L = 8192 example of the page
"AI Infra 第5章图解: 算子与运行时", section "FlashAttention: Softmax 也能逐块算").
Inputs are drawn once and resident in HBM before timing starts. Warm-up: W untimed steps,
continued until at least 0.2 s of GPU work has run (the clocks settle under the load),
reported as warmup_steps_run.

Printed: one JSON line with the throughput in algorithmic TFLOP/s over the timed steps
(2*(d+dv) per allowed query/key pair, softmax not counted; wall clock, nothing
instrumented); the roofline of the dominant kernel: its own launch duration, stamped at
the kernel's start and end by HIP events attached to each dispatch on the stream it is
launched on (the library's launch timer), as the mean, median, p10 and p90 over at least
50 back-to-back launches (warm) and over as many launches each after a 1 GiB cache flush
(cold), against the published peak and against the ceilings the library's probes measure
on this device (streaming copy for B_max, bf16 MFMA chains for P_max); the step period
(HIP events around the timed steps, which adds the gap between consecutive kernels); and
the CPU oracle timed on this host as a reported baseline (all threads, and one thread for
a per-core figure).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
  python bench.py --pass bwd [...]  # the gradients (fa_bwd) of the same workload instead
  python bench.py --tile-sweep      # tile shapes of the general kernel (fp32 experiment)
  python bench.py --copy-probe      # plain copy kernel of known size (counter calibration)
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

METRIC = "attention fwd TFLOP/s at N=8192,d=128 bf16 causal; % of MI355X MFMA peak"
# the other workloads name themselves in config.workload
OTHER_METRIC = "attention fwd TFLOP/s; % of MI355X MFMA peak"
DEFAULT_WORKLOAD = "bf16_causal_single_head_n8192_d128"
KERNEL_SRC = os.path.join(ROOT, "exact_attention_35_amd", "csrc", "fa_fwd_mfma.hip")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_sha(src: str = KERNEL_SRC) -> str:
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def read_traffic(workload: str, kind: str = "fwd_mfma", src: str = KERNEL_SRC):
    """HBM bytes per launch (forward) or per call (gradients, all their kernels) from a
    committed counter summary, if it was taken on the current kernel source; otherwise
    None."""
    path = os.path.join(PROFILES, f"traffic_{kind}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_sha(src):
        return None
    try:
        return float(kv["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def launch_stats(launch, stream, reps, flush=None):
    """Device time of `reps` launches, each bracketed by its own pair of HIP events on
    `stream` (the stream the library launches on). With `flush`, that untimed work runs
    on the stream before every launch (a cold-cache run). Returns the sorted times (s).
    Each time includes the gap between the start event and the kernel's start."""
    import numpy as np
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record(stream)
        launch()
        e1.record(stream)
    torch.cuda.synchronize()
    return np.sort(np.array([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e-3)


def kernel_stats(launch, reps, flush=None):
    """Durations of the main kernel in `reps` calls of `launch`, from the library's launch
    timer: each launch's own dispatch stamps its pair of events at the kernel's start and
    end, the interval a kernel-trace profiler reports. With `flush`, that untimed work runs
    before every call (a cold-cache run). Returns the sorted times (s)."""
    import numpy as np

    from exact_attention_35_amd import capi

    capi.fa_probe_timer_arm(reps)
    for _ in range(reps):
        if flush is not None:
            flush()
        launch()
    return np.sort(np.array(capi.fa_probe_timer_read(reps)) * 1e-6)


WARMUP_MIN_S = 0.2


def warm_up(step, steps, min_s=WARMUP_MIN_S):
    """Untimed warm-up: `steps` steps, continued in batches of 16 until at least `min_s`
    seconds of GPU work have passed. Under a new load the GPU's clocks take tens of
    milliseconds to settle: on the headline workload 20 warm-up steps leave the step period
    at 30.4-31.3 us and the kernel at 27.5 us, 2000 steps at 27.0 and 26.4 us. Returns the
    number of steps run."""
    import torch

    t0 = time.perf_counter()
    n = 0
    for _ in range(steps):
        step()
        n += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_s:
        for _ in range(16):
            step()
        n += 16
        torch.cuda.synchronize()
    return n


def timed_region(step, stream, steps):
    """The timed steps: wall clock around them, synchronised on both sides (`value`), and a
    pair of HIP events on the library's stream around the same steps (the step period).
    Nothing in them is instrumented. Returns (wall s, event s)."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) * 1e-3


def summary_us(t):
    """Median, p10, p90 and mean of launch times t (s), in microseconds."""
    import numpy as np

    return {"median": float(np.median(t)) * 1e6, "p10": float(np.percentile(t, 10)) * 1e6,
            "p90": float(np.percentile(t, 90)) * 1e6, "mean": float(np.mean(t)) * 1e6, "n": int(len(t))}


def make_flush(dev, stream, nbytes=1 << 30):
    """Untimed cache flush for cold runs: read and write a 1 GiB buffer (four times the
    256 MB last-level cache, so neither the L2s nor the Infinity Cache keep the inputs)."""
    import torch

    buf = torch.zeros(nbytes // 4, dtype=torch.float32, device=dev)

    def flush():
        with torch.cuda.stream(stream):
            buf.add_(1.0)
    return flush


def issue_probe():
    """The issue probe of include/fa_probe.h on every CU: cycles per MFMA of an MFMA wave
    with K vector ops (or E exponentials) after each MFMA, one wave per SIMD; and, with two
    waves per SIMD, an MFMA wave beside a vector-ALU wave, each alone and together, and two
    vector-ALU waves. Cycles are the shader clock's (s_memtime); MHz from s_memrealtime."""
    import torch

    from exact_attention_35_amd import capi

    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    iters = 20000

    def run(role, k, e):
        capi.fa_probe_issue(role, k, e, cus, iters)
        cyc, rt, waves = capi.fa_probe_issue(role, k, e, cus, iters)
        return cyc, waves, 100.0 * sum(cyc) / max(sum(rt), 1)

    rows = []
    for k, e in ((0, 0), (2, 0), (4, 0), (6, 0), (8, 0), (12, 0), (0, 1), (0, 2), (0, 4), (4, 1), (4, 2)):
        cyc, _, mhz = run(0, k, e)
        rows.append({"waves_per_simd": 1, "mfma_wave": {"valu_ops_per_mfma": k, "exps_per_mfma": e,
                                                        "cycles_per_mfma": sum(cyc) / len(cyc) / (2 * iters)},
                     "MHz": mhz})
    for e in (0, 1):
        ops = 4 if e else 12
        kind = "v_exp_f32" if e else "v_fma_f32"
        for role, what in ((2, "MFMA wave alone"), (3, "VALU wave alone"), (1, "MFMA wave beside a VALU wave"),
                           (4, "two VALU waves")):
            cyc, waves, mhz = run(role, 0, e)
            mf = [c for c, w in zip(cyc, waves) if role != 4 and w % 8 < 4]
            va = [c for c, w in zip(cyc, waves) if role == 4 or w % 8 >= 4]
            row = {"waves_per_simd": 2, "case": what, "valu_op": kind, "MHz": mhz}
            if mf:
                row["cycles_per_mfma"] = sum(mf) / len(mf) / (2 * iters)
            if va:
                row["cycles_per_valu_op_per_wave"] = sum(va) / len(va) / (iters * ops)
            rows.append(row)
    print(json.dumps({"probe": "issue", "device_cus": cus, "iters": iters, "rows": rows}), flush=True)
    return 0


def loop_probe():
    """The LDS probe and the tile-body probe of include/fa_probe.h on every CU, two
    workgroups of four waves per CU as the attention kernel runs: bytes per clock per CU of
    each LDS access kind, and shader cycles per tile for a SIMD's pair of waves running the
    forward kernel's tile instruction mix, without and with the tile's K/V copies. A
    launch's cycles are its duration (events around it, the second of two launches) times
    the mean shader clock of its waves (s_memtime over s_memrealtime)."""
    import torch

    from exact_attention_35_amd import capi

    dev = torch.device("cuda", torch.cuda.current_device())
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 2 * cus

    def cycles(res):
        cyc, rt, ms = res
        mhz = 100.0 * sum(cyc) / max(sum(rt), 1)
        return ms * 1e3 * mhz, mhz

    lds = []
    iters = 2000
    for mode, kind, width in ((0, "ds_read_b128", 16), (1, "ds_read_b64", 8), (2, "ds_read_b64_tr_b16", 8),
                              (3, "ds_read_b32", 4), (4, "ds_write_b128", 16)):
        capi.fa_probe_lds(mode, blocks, iters)
        c, mhz = cycles(capi.fa_probe_lds(mode, blocks, iters))
        total = blocks * 4 * iters * 8 * 64 * width
        lds.append({"access": kind, "bytes_per_clk_per_cu": round(total / c / cus, 1), "MHz": round(mhz)})
    src = torch.zeros(1 << 18, dtype=torch.uint8, device=dev)
    tiles = 400
    tile = []
    for copies, valu in ((0, 0), (0, 117), (1, 0), (1, 117)):
        capi.fa_probe_tile(copies, valu, blocks, tiles, src)
        c, mhz = cycles(capi.fa_probe_tile(copies, valu, blocks, tiles, src))
        tile.append({"copies": copies, "valu_ops": valu, "exps": 33, "cycles_per_tile_pair": round(c / tiles),
                     "MHz": round(mhz)})
    print(json.dumps({"probe": "loop", "device_cus": cus, "lds": lds, "tile": tile,
                      "mfma_bound_cycles_per_tile_pair": 2 * 32 * 32}), flush=True)
    return 0


def measured_ceilings(dev, stream):
    """B_max from the library's streaming copy probe (2 GiB each way, far beyond the last-level
    cache) and from its read-only probe (the same 2 GiB read), and the bf16 matrix-core
    ceiling from its MFMA probe (two workgroups of four waves per compute unit, as the
    attention kernel runs), each the median over 20 launches."""
    import torch

    from exact_attention_35_amd import capi

    n = 2 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        capi.fa_probe_copy(src, dst, stream)
    t = launch_stats(lambda: capi.fa_probe_copy(src, dst, stream), stream, 20)
    bw = 2.0 * n / float(t[len(t) // 2])
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(16 * cus, dtype=torch.int32, device=dev)
    for _ in range(3):
        capi.fa_probe_read(src, sink, stream)
    t = launch_stats(lambda: capi.fa_probe_read(src, sink, stream), stream, 20)
    rbw = n / float(t[len(t) // 2])
    del src, dst
    blocks, iters = 2 * cus, 4000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    flops = capi.fa_probe_mfma(out, blocks, iters, stream)
    t = launch_stats(lambda: capi.fa_probe_mfma(out, blocks, iters, stream), stream, 20)
    return {"hbm_GBps": bw / 1e9, "hbm_read_GBps": rbw / 1e9, "mfma_bf16_TFLOPs": flops / float(t[len(t) // 2]) / 1e12,
            "copy_probe_bytes": 2 * n, "read_probe_bytes": n,
            "mfma_probe": f"{blocks} workgroups x 4 waves x {iters} x 4 MFMA 32x32x16"}


def cpu_host_info():
    """The host's CPU model, the cores this process may use and the BLAS threads."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads = None
    try:
        from threadpoolctl import threadpool_info

        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": threads}


def copy_probe(steps: int) -> None:
    """A plain elementwise copy kernel (x * 1 -> y, fp32) over 256 MiB, `steps` times:
    its FETCH_SIZE / WRITE_SIZE readings calibrate those counters against a known
    256 MiB read and 256 MiB write per dispatch."""
    import torch

    n = (256 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "steps": steps}))


def cpu_baseline(w, inp, budget_s=10.0):
    """Time the fp64 oracle on this host's cores for about `budget_s` seconds.

    Workloads whose dense score matrix the oracle builds in a few seconds are run whole,
    repeatedly, until the budget is spent; larger ones are timed on whole query rows of
    head (0, 0) (every key of each row, as the definition computes it), as many rows as
    fit the budget, and the rate is taken over those rows' algorithmic FLOPs.
    """
    import numpy as np

    from exact_attention_35_amd import roofline as rf
    from oracle import sdpa_reference, sdpa_reference_rows

    threads = None
    try:
        from threadpoolctl import threadpool_info

        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    dense = 2.0 * (w.d + w.dv) * w.n_q * w.N * w.B * w.H
    if dense <= 60e9:  # whole workload
        calls, total = 0, 0.0
        while total < budget_s and calls < 50:
            t0 = time.perf_counter()
            sdpa_reference(inp["q"], inp["k"], inp["v"], inp["bias"], w.causal)
            total += time.perf_counter() - t0
            calls += 1
        flops = rf.alg_flops(w.B, w.H, w.N, w.d, w.dv, w.causal, Nq=w.n_q) * calls
        sample = f"whole workload ({w.name}), {calls} call{'s' if calls != 1 else ''}, fp64 numpy, {total:.1f} s"
    else:  # whole rows of head (0, 0), spread over the sequence
        rng = np.random.default_rng(0)
        rows_done, flops, total = 0, 0, 0.0
        while total < budget_s and rows_done < w.N:
            rows = np.sort(rng.choice(w.N, size=min(64, w.N), replace=False))
            t0 = time.perf_counter()
            sdpa_reference_rows(inp["q"], inp["k"], inp["v"], inp["bias"], w.causal, 0, 0, rows)
            total += time.perf_counter() - t0
            keys = (rows + 1) if w.causal else np.full(len(rows), w.N)
            flops += int(2 * (w.d + w.dv) * keys.sum())
            rows_done += len(rows)
        sample = f"{rows_done} whole query rows of head (0, 0) of {w.name}, fp64 numpy, {total:.1f} s"
    res = {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": sample, "seconds": total, **cpu_host_info()}
    res["one_thread"] = cpu_baseline_one_thread(w, inp)
    return res


def cpu_baseline_one_thread(w, inp, budget_s=4.0):
    """The same oracle with BLAS held to one thread, on whole query rows of head (0, 0)
    (64 rows a call, spread over the sequence), for a per-core figure."""
    import numpy as np

    from oracle import sdpa_reference_rows

    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        return None
    rng = np.random.default_rng(1)
    flops, total, done = 0, 0.0, 0
    with threadpool_limits(limits=1):
        while total < budget_s and done < w.n_q:
            rows = np.sort(rng.choice(w.n_q, size=min(64, w.n_q), replace=False))
            t0 = time.perf_counter()
            sdpa_reference_rows(inp["q"], inp["k"], inp["v"], inp["bias"], w.causal, 0, 0, rows)
            total += time.perf_counter() - t0
            off = w.N - w.n_q
            keys = np.minimum(rows + 1 + off, w.N) if w.causal else np.full(len(rows), w.N)
            flops += int(2 * (w.d + w.dv) * keys.sum())
            done += len(rows)
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": 1,
            "sample": f"{done} whole query rows of head (0, 0), BLAS limited to one thread, {total:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--reps", type=int, default=50,
                    help="individually timed launches, warm and cold each (at least --steps)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the copy and MFMA probes (e.g. under a counter profiler)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--issue-probe", action="store_true",
                    help="how one SIMD shares MFMA and vector-ALU issue (fa_probe_issue); prints one JSON line")
    ap.add_argument("--loop-probe", action="store_true",
                    help="LDS throughput and the tile-body model (fa_probe_lds, fa_probe_tile); prints one JSON line")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward (default) or the gradients of the workload")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="time the general kernel's tile shapes on the fp32 sweep workload")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported; this path has no multi-GPU mode", file=sys.stderr)
        return 2

    import torch

    if args.issue_probe:
        return issue_probe()
    if args.loop_probe:
        return loop_probe()
    if args.copy_probe:
        copy_probe(args.steps)
        return 0
    if args.tile_sweep:
        return tile_sweep(args)

    import numpy as np

    from exact_attention_35_amd import capi, roofline as rf, workloads

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    inp = workloads.make_inputs(w, device="cpu")
    gpu = {}
    for n, t in inp.items():
        if t is None:
            gpu[n] = None
        elif w.layout == "bnhd" and n in ("q", "k", "v"):
            gpu[n] = t.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
        else:
            gpu[n] = t.to(dev)
    out = torch.empty(w.B, w.H, w.n_q, w.dv, dtype=gpu["q"].dtype, device=dev)
    lse = torch.empty(w.B, w.H, w.n_q, dtype=torch.float32, device=dev)
    if args.which == "bwd":
        return bench_bwd(args, w, inp, gpu, out, lse)

    # One validated call through the binding, then the same C entry point with its
    # arguments marshalled once, so the timed loop is the library call itself. Workloads
    # with N_q query rows against N keys go through fa_fwd_qk.
    rect = w.n_q != w.N
    if rect:
        capi.fa_fwd_qk(gpu["q"], gpu["k"], gpu["v"], bias=gpu["bias"], causal=w.causal, out=out, lse=lse)
    else:
        capi.fa_fwd(gpu["q"], gpu["k"], gpu["v"], bias=gpu["bias"], causal=w.causal, out=out, lse=lse)
    stream = torch.cuda.current_stream(dev)   # fa_fwd launches on this stream
    L = capi.lib()
    strides = capi.make_strides(gpu["q"], gpu["k"], gpu["v"], out,
                                None if gpu["bias"] is None else gpu["bias"].expand(w.B, w.H, w.n_q, w.N),
                                lse)
    vp = ctypes.c_void_p
    sizes = (w.B, w.H, w.n_q, w.N) if rect else (w.B, w.H, w.N)
    call = (vp(gpu["q"].data_ptr()), vp(gpu["k"].data_ptr()), vp(gpu["v"].data_ptr()),
            vp(0 if gpu["bias"] is None else gpu["bias"].data_ptr()),
            capi.FA_MASK_CAUSAL if w.causal else capi.FA_MASK_NONE,
            vp(out.data_ptr()), vp(lse.data_ptr()), *sizes, w.d, w.dv,
            ctypes.byref(strides), capi.FA_BF16 if w.dtype == "bf16" else capi.FA_F32,
            vp(stream.cuda_stream))
    entry = L.fa_fwd_qk if rect else L.fa_fwd

    def step():
        st = entry(*call)
        if st:
            raise capi.FaError(st, capi.fa_status_string(st))

    warmed = warm_up(step, args.warmup)

    # the timed steps: wall clock (`value`) and HIP events on the library's stream around
    # them (the step period: the kernel plus the gap before the next one starts)
    wall, ev_s = timed_region(step, stream, args.steps)
    # the kernel's own launch duration: the timed steps again, back to back, each launch
    # stamped at its start and end by its dispatch (warm), and the same after a 1 GiB flush
    # (cold); stamping adds work between launches, so it stays out of the timed steps
    reps = max(args.reps, args.steps)
    warm = kernel_stats(step, reps)
    cold = kernel_stats(step, reps, flush=make_flush(dev, stream))
    ceil = {"hbm_GBps": None, "mfma_bf16_TFLOPs": None} if args.no_ceilings else measured_ceilings(dev, stream)

    flops = rf.alg_flops(w.B, w.H, w.N, w.d, w.dv, w.causal, Nq=w.n_q)
    elem = 2 if w.dtype in ("bf16", "f16") else 4
    bias_bytes = (w.H * w.n_q * w.N * 4) if w.bias else 0
    min_b = rf.min_bytes(w.B, w.H, w.N, w.d, w.dv, elem, bias_bytes=bias_bytes, Nq=w.n_q)
    value = flops * args.steps / wall / 1e12
    period = ev_s / args.steps
    avg = float(np.mean(warm))
    med_w, med_c = float(np.median(warm)), float(np.median(cold))
    # the ceiling of the kernel that runs: bf16 on the matrix cores; fp32 on the general
    # kernel's vector ALUs
    mfma = w.dtype in ("bf16", "f16")
    peak = (rf.MI355X_PEAK_BF16_FLOPS if mfma else rf.MI355X_PEAK_F32_FLOPS) / 1e12
    bound = "mfma" if mfma else "alu"
    # which ceiling binds at I = F/Q: the bias stream (and a decoding step, which reads
    # every key and value for one row) make a workload memory-bound
    _, _, which = rf.roofline_bound(flops, min_b, peak * 1e12, rf.MI355X_HBM_BYTES_PER_S)
    if which == "memory":
        bound = "hbm"
    traffic = read_traffic(w.name)
    if bound == "hbm":
        meas = ceil["hbm_GBps"]
        rate = lambda t: min_b / t / 1e9
        roof = {"bound": "hbm", "peak": 8000.0, "unit": "GB/s"}
    else:
        meas = ceil["mfma_bf16_TFLOPs"] if mfma else None
        rate = lambda t: flops / t / 1e12
        roof = {"bound": bound, "peak": peak, "unit": "TFLOP/s"}
    roof.update({"achieved": rate(avg), "frac": rate(avg) / roof["peak"], "traffic": traffic,
                 "median_achieved": rate(med_w), "median_frac": rate(med_w) / roof["peak"],
                 "measured_peak": meas, "frac_of_measured": (rate(avg) / meas) if meas else None,
                 "cold_achieved": rate(med_c), "cold_frac": rate(med_c) / roof["peak"]})
    # the attainable rate on the measured ceilings, min(P_max, B_max * I) with I = FLOPs per
    # minimum byte (matrix-core kernels: P_max from the MFMA probe, B_max from the copy probe)
    # (B_max: the read-only probe's bandwidth for kernels whose minimum bytes are at least 90%
    # reads, as a decoding step and the bias stream are; else the copy probe's)
    if mfma and ceil["mfma_bf16_TFLOPs"] and ceil["hbm_GBps"]:
        p_max = ceil["mfma_bf16_TFLOPs"]
        writes = w.B * w.H * w.n_q * (w.dv * elem + 4)
        reads_share = 1.0 - writes / min_b
        b_src = "read probe" if reads_share >= 0.9 and ceil.get("hbm_read_GBps") else "copy probe"
        b_max = ceil["hbm_read_GBps"] if b_src == "read probe" else ceil["hbm_GBps"]
        b_i = b_max * 1e9 * (flops / min_b) / 1e12
        attain = min(p_max, b_i)
        roof["measured_roofline"] = {"P_max_TFLOPs": p_max, "B_max_GBps": b_max, "B_max_source": b_src,
                                     "read_share_of_min_bytes": reads_share, "B_max_x_I_TFLOPs": b_i,
                                     "intensity_flop_per_byte": flops / min_b, "attainable_TFLOPs": attain,
                                     "achieved_TFLOPs": flops / avg / 1e12, "frac": flops / avg / 1e12 / attain,
                                     "bound": "mfma" if p_max <= b_i else "hbm"}
    roof.update({"kernel": "fwd_mfma" if mfma else "fwd_generic",
                 "avg_launch_us": avg * 1e6, "step_period_us": period * 1e6,
                 "launch_us_warm": summary_us(warm), "launch_us_cold": summary_us(cold),
                 "timing": ("avg_launch_us / launch_us_warm: the kernel's own start/end stamps (HIP events "
                            "that hipExtLaunchKernelGGL attaches to the dispatch, on the library's stream) "
                            "over max(reps, steps) back-to-back repeats of the timed step; launch_us_cold: "
                            "the same after a 1 GiB flush each; step_period_us: HIP events around the "
                            "uninstrumented timed steps, per step (adds the gap between consecutive kernels)"),
                 "alg_flops_per_launch": flops, "min_bytes_per_launch": min_b,
                 "measured_ceilings": ceil,
                 "kernel_source_sha256_16": kernel_sha()})
    ws_bytes = capi.fa_fwd_qk_workspace_size(w.B, w.H, w.n_q, w.N, w.d, w.dv,
                                             capi.FA_BF16 if w.dtype == "bf16" else capi.FA_F32, w.causal)

    res = {
        "metric": METRIC if args.workload == DEFAULT_WORKLOAD else OTHER_METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warmed,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dv": w.dv,
                   "causal": w.causal, "bias": w.bias, "layout": w.layout,
                   "parallelism": "single GPU", "workspace_bytes": int(ws_bytes),
                   **({"N_q": w.n_q} if rect else {})},
        "pct_of_peak": 100.0 * value / peak,
        "roofline": roof,
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(res), flush=True)
    return 0


# (FA_GENERIC_TILE value, query rows per workgroup BM, keys per block BK)
TILES = [(1, 32, 32), (0, 64, 32), (2, 64, 16), (3, 64, 64), (4, 128, 32)]


def tile_sweep(args) -> int:
    """The tile-shape experiment: the general fp32 kernel at each (BM, BK) on one
    workload; one JSON line per tile with the time per call and the modelled bytes that
    the workgroups load (every query tile streams all N keys and values once:
    B*H * ceil(N/BM) * N * (d + dv) * 4 bytes, the pages' N^2 d^2 / M with BM ~ M / d)."""
    import torch

    from exact_attention_35_amd import capi, roofline as rf, workloads

    w = workloads.WORKLOADS["fp32_tile_sweep_h8_n4096_d64"]
    dev = torch.device("cuda:0")
    g = {n: (None if t is None else t.to(dev)) for n, t in workloads.make_inputs(w).items()}
    for code, bm, bk in TILES:
        os.environ["FA_GENERIC_TILE"] = str(code)
        f = lambda: capi.fa_fwd(g["q"], g["k"], g["v"], causal=w.causal)  # noqa: E731
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        kv_bytes = w.B * w.H * (-(-w.N // bm)) * w.N * (w.d + w.dv) * 4
        flops = rf.alg_flops(w.B, w.H, w.N, w.d, w.dv, w.causal)
        print(json.dumps({"tile_sweep": w.name, "BM": bm, "BK": bk, "FA_GENERIC_TILE": code,
                          "us_per_call": us, "TFLOP/s": flops / us / 1e6,
                          "model_kv_load_bytes": kv_bytes}), flush=True)
    os.environ.pop("FA_GENERIC_TILE", None)
    return 0


BWD_METRIC = "attention bwd (dQ, dK, dV) TFLOP/s; % of MI355X MFMA peak"
BWD_SRC = os.path.join(ROOT, "exact_attention_35_amd", "csrc", "fa_bwd_mfma.hip")


def cpu_baseline_bwd(w, inp, budget_s=10.0):
    """Time the fp64 gradient oracle on this host for about `budget_s` seconds: the whole
    workload when its dense score matrix is small, else head (0, 0) alone, repeated."""
    from exact_attention_35_amd import roofline as rf
    from oracle import sdpa_backward_reference

    try:
        from threadpoolctl import threadpool_info

        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        threads = None
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    whole = w.B * w.H == 1 or 2.0 * (3 * w.d + 2 * w.dv) * w.N * w.N * w.B * w.H <= 60e9
    sl = (slice(None),) * 2 if whole else (slice(0, 1), slice(0, 1))
    bias = inp["bias"]
    if bias is not None and not whole:
        bias = bias[:1, :1]
    args = [inp[n][sl] for n in ("q", "k", "v", "do")]
    calls, total = 0, 0.0
    while total < budget_s and calls < 50:
        t0 = time.perf_counter()
        sdpa_backward_reference(*args, bias, w.causal)
        total += time.perf_counter() - t0
        calls += 1
    bh = w.B * w.H if whole else 1
    flops = rf.alg_flops_bwd(1, bh, w.N, w.d, w.dv, w.causal) * calls
    what = f"whole workload ({w.name})" if whole else f"head (0, 0) of {w.name}"
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what}, {calls} call{'s' if calls != 1 else ''}, fp64 numpy, {total:.1f} s",
            "seconds": total}


def bench_bwd(args, w, inp, gpu, out, lse) -> int:
    """A step is one fa_bwd call (row statistics + gradient kernel) on the workload,
    with O and lse from one fa_fwd call and a seeded dO, all resident in HBM."""
    import torch

    import numpy as np

    from exact_attention_35_amd import capi, roofline as rf, workloads

    if w.dtype != "bf16":
        print("the gradients are implemented for bf16 workloads only", file=sys.stderr)
        return 2
    dev = gpu["q"].device
    inp["do"] = workloads.make_grad_out(w, device="cpu")
    do = inp["do"]
    if w.layout == "bnhd":
        do = do.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
    else:
        do = do.to(dev)
    capi.fa_fwd(gpu["q"], gpu["k"], gpu["v"], bias=gpu["bias"], causal=w.causal, out=out, lse=lse)
    dq = torch.empty_like(gpu["q"])
    dk = torch.empty_like(gpu["k"])
    dv = torch.empty_like(gpu["v"])
    stream = torch.cuda.current_stream(dev)

    def step():
        capi.fa_bwd(gpu["q"], gpu["k"], gpu["v"], out, lse, do, bias=gpu["bias"], causal=w.causal,
                    grad_q=dq, grad_k=dk, grad_v=dv, stream=stream)

    warmed = warm_up(step, args.warmup)
    # the timed steps: wall clock (`value`) and HIP events around them on the library's
    # stream (the average fa_bwd call, all its kernels)
    wall, ev_s = timed_region(step, stream, args.steps)
    avg_call_s = ev_s / args.steps
    # one fa_bwd call (all its kernels) bracketed by its own events, warm and cold; and
    # the dK/dV/dQ kernel alone, from its own start/end stamps
    reps = max(args.reps, args.steps)
    flush = make_flush(dev, stream)
    warm = launch_stats(step, stream, reps)
    cold = launch_stats(step, stream, reps, flush=flush)
    main_warm = kernel_stats(step, reps)
    main_cold = kernel_stats(step, reps, flush=flush)

    flops = rf.alg_flops_bwd(w.B, w.H, w.N, w.d, w.dv, w.causal)
    peak = rf.MI355X_PEAK_BF16_FLOPS / 1e12
    achieved = flops / avg_call_s / 1e12
    bias_bytes = (w.H * w.N * w.N * 4) if w.bias else 0
    res = {
        "metric": BWD_METRIC,
        "value": flops * args.steps / wall / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warmed,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs and dO of the workload's shape)",
        "config": {"workload": w.name, "pass": "bwd", "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dv": w.dv,
                   "causal": w.causal, "bias": w.bias, "layout": w.layout, "parallelism": "single GPU",
                   "workspace_bytes": int(capi.fa_bwd_workspace_size(w.B, w.H, w.N, w.d, w.dv, capi.FA_BF16,
                                                                     w.causal))},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": read_traffic(w.name, "bwd", BWD_SRC),
                     "cold_achieved": flops / float(np.median(cold)) / 1e12,
                     "cold_frac": flops / float(np.median(cold)) / 1e12 / peak,
                     "kernel": "bwd_rowstat + bwd_mfma [+ bwd_reduce] (one fa_bwd call)",
                     "avg_launch_us": avg_call_s * 1e6, "launch_us_warm": summary_us(warm),
                     "launch_us_cold": summary_us(cold),
                     "main_kernel_us_warm": summary_us(main_warm), "main_kernel_us_cold": summary_us(main_cold),
                     "timing": ("avg_launch_us: HIP events on the library's stream around the timed calls, "
                                "per call; launch_us_*: one call between its own pair of events; "
                                "main_kernel_us_*: bwd_mfma's own start/end stamps (hipExtLaunchKernelGGL events)"),
                     "alg_flops_per_launch": flops,
                     "min_bytes_per_launch": rf.min_bytes_bwd(w.B, w.H, w.N, w.d, w.dv, 2, bias_bytes),
                     "kernel_source_sha256_16": hashlib.sha256(open(BWD_SRC, "rb").read()).hexdigest()[:16]},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline_bwd(w, inp)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
