"""Throughput of the Longformer window + global attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qa_4k]

One step = one forward pass (two kernels: the band kernel -- window band,
global-column fold, global-row partials -- and the log-sum-exp merge of those
partials) over one batch of seeded synthetic input already resident in HBM.  The
metric is effective TFLOP/s: 4*d_h FLOP per attended (query, key) pair, pairs counted
exactly (window + globals after de-duplication and padding), divided by the wall time
of the K timed steps.  Before the W warm-up steps, steps run back to back for at least
--clock-warmup seconds (the GPU clock ramps up under load).

Prints one JSON line.  Also reported: the band kernel's own rate against the bf16
MFMA peak (each launch stamped with the kernel's start and end by HIP events on the
launch stream), and the fp64 CPU oracle timed on a bounded sample of the same
workload on the host's cores.

Variants (not the default line): --global-proj (separate projections of the global
rows; with --backward its backward), --backward (the backward pass alone and a
forward + backward training step).
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

# MI355X: 256 CUs x 2.4 GHz x 4096 bf16 FLOP/clk/CU (dense), HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
METRIC = "window+global attn fwd effective TFLOP/s and % bf16 MFMA peak, L=4096 w=512"
CSRC = os.path.join(ROOT, "sparse_long_sequence_longformer_amd", "csrc")
# Sources of the forward kernels (the traffic counters are valid for this text only).
KERNEL_SRCS = [os.path.join(CSRC, f) for f in ("lf_attn_kernels.hip", "lf_attn_device.h", "lf_attn_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "band_kernel_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU clock settles after about 0.1 s of back-to-back steps (~1500 steps of the
    # L=4096 workload); the defaults warm up past that and time a comparable span.
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--clock-warmup", type=float, default=0.3, metavar="SECONDS",
                    help="back-to-back steps for at least this long before the --warmup steps")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--global-proj", action="store_true",
                    help="global rows use their own q/k/v projections (lf_attn_forward_global_proj)")
    ap.add_argument("--causal", action="store_true",
                    help="one-sided variant: no pair with its key after its query")
    ap.add_argument("--bias", type=float, default=0.0, metavar="SCALE",
                    help="relative position bias on window scores: a seeded N(0, SCALE^2) table per head "
                         "(0: none)")
    ap.add_argument("--random", type=int, default=0, metavar="R",
                    help="BigBird-style random attention: R seeded key blocks of 64 per (head, query block) "
                         "(0: none; needs an undilated workload)")
    ap.add_argument("--layer", action="store_true",
                    help="time one whole layer (projections, attention, LayerNorms, GELU feed-forward)")
    ap.add_argument("--ffn", type=int, default=3072, help="feed-forward width of --layer")
    ap.add_argument("--graph", action="store_true",
                    help="also time the forward captured in a HIP graph and replayed")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (lf_attn_backward) instead of the forward")
    ap.add_argument("--tile-rows", type=int, default=0, choices=(0, 64, 128),
                    help="forward rows per work-group (lf_attn_set_tile_rows; 0: the library chooses)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--trials", type=int, default=15, help="timing trials after the main window (median/min/p90)")
    ap.add_argument("--trial-steps", type=int, default=500, help="steps per timing trial")
    ap.add_argument("--cold-trials", type=int, default=20,
                    help="single steps each after writing 512 MiB elsewhere (evicts the 256 MB Infinity Cache)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    return ap.parse_args()


def traffic_for(workload: str):
    """HBM bytes per band-kernel launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_sha") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, q, k, v, G, pad, target_s, causal=False, bias=None, rand=None):
    """The fp64 oracle on whole (b, h) slices of the workload, on a pool of host threads
    (one per core of this process's CPU share, at most 16; BLAS limited to one thread
    per call, numpy's array work runs outside the interpreter lock).  Slices are handed
    out in order until about target_s seconds have passed; the slices finished count."""
    from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait

    from threadpoolctl import threadpool_limits

    from oracle import longformer_oracle as orc
    from sparse_long_sequence_longformer_amd import pattern

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    slices = [(b, h) for b in range(wl.B) for h in range(wl.H)]

    def one(b, h):
        orc.attention_bh(q[b, h], k[b, h], v[b, h], wl.w, wl.dil[h], G, None if pad is None else pad[b],
                         causal=causal, bias=None if bias is None else bias[h],
                         rand=None if rand is None else rand[h])
        pr = None if pad is None else pad[b:b + 1]
        return pattern.count_pairs(wl.L, wl.w, [wl.dil[h]], G, pr, causal=causal,
                                   rand=None if rand is None else [rand[h]]).total

    pairs = 0
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1), ThreadPoolExecutor(threads) as ex:
        nxt = 0
        running = set()
        while nxt < len(slices) or running:
            while nxt < len(slices) and len(running) < threads and time.perf_counter() - t0 < target_s:
                running.add(ex.submit(one, *slices[nxt]))
                nxt += 1
            if not running:
                break
            fin, running = wait(running, return_when=FIRST_COMPLETED)
            for f in fin:
                pairs += f.result()
                done += 1
    dt = time.perf_counter() - t0
    return {
        "value": 256.0 * pairs / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {wl.B * wl.H} (batch, head) slices of {wl.name}, full rows, {dt:.1f} s wall on "
                  f"{threads} threads; same effective-FLOP count as the GPU value",
        "cpu_model": cpu_model(),
        "seconds": round(dt, 3),
        "pairs": pairs,
    }


def clock_warmup(step, seconds, torch):
    """Back-to-back steps until at least `seconds` have passed (the GPU clock ramps up
    over about the first 0.1 s of load), ahead of the requested warm-up steps.
    Returns (seconds spent, steps run)."""
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(50):
            step()
        n += 50
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return round(time.perf_counter() - t0, 3), n


def split_tiling(wl, args) -> bool:
    """Whether the library runs this forward on 64-row split work-groups: its rule for
    a handle left at tile rows 0 (the 128-row grid fills at most half of the
    work-group slots, three bf16 or one fp32 work-group per compute unit; never with a
    position bias or random blocks)."""
    import torch

    if args.bias or args.random or args.layer or args.tile_rows == 128:
        return False
    if args.tile_rows == 64:
        return True
    tiles = 0
    for d in wl.dil_list():
        tiles = max(tiles, d * (((wl.L + d - 1) // d + 127) // 128))
    slots = torch.cuda.get_device_properties(0).multi_processor_count * (3 if wl.dtype == "bf16" else 1)
    return 2 * wl.B * wl.H * tiles <= slots


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by (batch, head) or by sequence; no multi-GPU path is implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_long_sequence_longformer_amd import binding, pattern, workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    binding.load_library()
    dev = torch.device("cuda:0")

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 5}))
        return

    name = args.workload or workloads.HEADLINE
    wl = workloads.WORKLOADS[name]
    q, k, v = workloads.make_qkv(wl)
    G = wl.global_positions()
    pad = wl.pad_mask()
    rand_tab = None
    if args.random:
        if any(d != 1 for d in wl.dil_list()):
            print("bench.py: --random needs an undilated workload", file=sys.stderr)
            sys.exit(2)
        rand_tab = workloads.make_random_blocks(wl.H, wl.L, args.random, seed=wl.seed)
    pairs = pattern.count_pairs(wl.L, wl.w, wl.dil_list(), G, pad, B=wl.B, causal=args.causal, rand=rand_tab)
    flops = pattern.effective_flops(pairs.total)

    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    padd = None if pad is None else torch.from_numpy(pad).to(dev)
    out = torch.empty_like(qd)
    handle = binding.LfAttn(wl.dtype)
    handle.set_tile_rows(args.tile_rows)
    if args.causal:
        handle.set_causal(True)
    bias_tab = None
    if args.bias:
        bias_tab = workloads.make_bias(wl.H, wl.w, seed=wl.seed, scale=args.bias)
        handle.set_position_bias(torch.from_numpy(bias_tab).to(dev))
    if rand_tab is not None:
        handle.set_random_blocks(rand_tab)
    dil = wl.dil_list()

    # One checked call through the Python wrapper, then the timed loops call the C entry
    # point with arguments marshalled once (the wrapper's checks cost host time that
    # is not part of the method).
    import ctypes

    lib = binding.load_library()
    i32p = ctypes.POINTER(ctypes.c_int32)
    dil_arr = (ctypes.c_int32 * len(dil))(*dil)
    g_arr = (ctypes.c_int32 * max(1, len(G)))(*G)
    tail = (wl.B, wl.H, wl.L, wl.d, wl.w, ctypes.cast(dil_arr, i32p), ctypes.cast(g_arr, i32p), len(G),
            None if padd is None else padd.data_ptr(), torch.cuda.current_stream().cuda_stream)
    if args.global_proj:
        qgd, kgd, vgd = (t.to(dev) for t in workloads.make_global_proj(wl))
        binding.forward_global_proj(qd, kd, vd, qgd, kgd, vgd, wl.w, dil, G, padd, out=out, handle=handle,
                                    causal=args.causal)
        fn = lib.lf_attn_forward_global_proj
        cargs = (handle.handle, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), qgd.data_ptr(), kgd.data_ptr(),
                 vgd.data_ptr(), out.data_ptr()) + tail
    else:
        binding.forward(qd, kd, vd, wl.w, dil, G, padd, out=out, handle=handle, causal=args.causal)
        fn = lib.lf_attn_forward
        cargs = (handle.handle, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr()) + tail

    def step():
        if fn(*cargs) != 0:
            raise RuntimeError(lib.lf_attn_last_error(handle.handle).decode())

    if args.layer:
        return bench_layer(args, wl, name, padd, G, dil, flops, handle)
    if args.backward:
        if wl.dtype != "bf16":
            print("bench.py: the backward runs on bf16 workloads only", file=sys.stderr)
            sys.exit(2)
        gp = (qgd, kgd, vgd) if args.global_proj else None
        return bench_backward(args, wl, name, qd, kd, vd, padd, G, dil, pairs, flops, handle, gp)

    clock = clock_warmup(step, args.clock_warmup, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    value = flops / (ms_step * 1e-3) / 1e12

    # Per-kernel durations over a second run of K steps: every kernel is launched with
    # a pair of HIP events that the launch itself stamps with the kernel's start and end
    # (hipExtLaunchKernel, on the launch stream).
    handle.set_stage_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    st = handle.stage_times()
    handle.set_stage_timing(False)
    stage_avg = {k2: v2[0] / v2[1] for k2, v2 in st.items() if v2[1]}
    k_avg_ms = stage_avg["band"]  # the dominant kernel
    traffic = None if (args.global_proj or args.causal or args.bias or args.random) else traffic_for(name)

    # Trials (median / min / p90 of per-step time) and cold steps (Infinity Cache evicted).
    def timed(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            step()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    trial_us = sorted(1e3 * timed(args.trial_steps) for _ in range(args.trials))
    cold_us = []
    if args.cold_trials:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for t in range(args.cold_trials):
            scratch.fill_(t & 0xFF)
            cold_us.append(1e3 * timed(1))
        del scratch
        cold_us.sort()

    def pct(xs, f):
        return round(xs[min(len(xs) - 1, int(f * (len(xs) - 1) + 0.5))], 3) if xs else None

    # Roofline of the dominant kernel: matrix cores above the ridge point (FLOP per byte
    # of the bf16 peak over the HBM peak), HBM below it.  Algorithmic bytes: Q, K, V read
    # and O written once (plus the pad mask).
    elem = 2 if wl.dtype == "bf16" else 4
    alg_bytes = 4 * wl.B * wl.H * wl.L * wl.d * elem + (0 if pad is None else wl.B * wl.L)
    if args.global_proj:
        alg_bytes += 3 * wl.B * wl.H * wl.L * wl.d * elem
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    mfma_bound = flops / alg_bytes >= ridge
    if mfma_bound:
        achieved = flops / (k_avg_ms * 1e-3) / 1e12  # every attended pair but the merge's arithmetic
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = alg_bytes / (k_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    t_roof_ms = max(flops / (PEAK_BF16_TFLOPS * 1e12), alg_bytes / (PEAK_HBM_GBS * 1e9)) * 1e3

    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_warmup_s": clock[0],
        "clock_warmup_steps": clock[1],
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, no trained weights)",
        "config": {
            "workload": name,
            "B": wl.B, "H": wl.H, "seq_len": wl.L, "d_h": wl.d, "w": wl.w,
            "dil": sorted(set(dil)), "n_global": len(G),
            "padded_lengths": list(wl.lengths) or None,
            "global_batch": wl.B,
            "parallelism": "single GPU",
            "global_projections": "separate" if args.global_proj else "shared",
            "window": "one-sided" if args.causal else "symmetric",
            "position_bias": f"N(0, {args.bias:g}^2) table" if args.bias else None,
            "random_blocks": f"{args.random} of 64 keys per (head, query block)" if args.random else None,
            "tile_rows": 64 if split_tiling(wl, args) else 128,
        },
        "pct_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 3),
        "attended_pairs": pairs.total,
        "effective_flop_per_step": flops,
        "kernel_ms_avg": {k2: round(v2, 6) for k2, v2 in stage_avg.items()},
        "roofline": {
            "kernel": f"lf::band_kernel<{'Bf16' if wl.dtype == 'bf16' else 'F32'}, {str(args.causal).lower()}, "
                      f"{str(bool(args.bias)).lower()}, {str(bool(args.random)).lower()}, false, "
                      f"{str(split_tiling(wl, args)).lower()}>",
            **roof,
            "traffic": traffic,
            "avg_launch_ms": round(k_avg_ms, 6),
            "avg_launch_source": "HIP events stamped by hipExtLaunchKernel with the kernel's own start and end, "
                                 "live over a second run of the timed steps",
            "flop_per_launch": flops,
            "alg_bytes_per_launch": alg_bytes,
            "arithmetic_intensity": round(flops / alg_bytes, 1),
        },
        "pct_of_roofline_time": round(100.0 * t_roof_ms / ms_step, 2),
        "us_per_step_trials": {"n": len(trial_us), "steps_each": args.trial_steps, "median": pct(trial_us, 0.5),
                               "min": pct(trial_us, 0.0), "p90": pct(trial_us, 0.9)},
        "us_per_step_cold": {"n": len(cold_us), "median": pct(cold_us, 0.5), "min": pct(cold_us, 0.0),
                             "p90": pct(cold_us, 0.9)},
        "env": {"numpy": np.__version__, "torch": torch.__version__},
    }
    if args.graph:
        # The same step captured once (the workspace already exists) and replayed.
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            if args.global_proj:
                binding.forward_global_proj(qd, kd, vd, qgd, kgd, vgd, wl.w, dil, G, padd, out=out, handle=handle,
                                            causal=args.causal)
            else:
                binding.forward(qd, kd, vd, wl.w, dil, G, padd, out=out, handle=handle, causal=args.causal)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        ms_g = a.elapsed_time(b) / args.steps
        res["graph_replay"] = {"ms_per_step": round(ms_g, 6), "value": round(flops / (ms_g * 1e-3) / 1e12, 3)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, q, k, v, G, pad, args.cpu_seconds, args.causal, bias_tab, rand_tab)
    print(json.dumps(res), flush=True)


def bench_layer(args, wl, name, padd, G, dil, flops_attn, handle):
    """One layer on the workload's shape (hidden = 64 * H) with seeded synthetic
    weights: the four GEMMs (hipBLASLt), the attention and the pointwise passes."""
    import ctypes

    import numpy as np
    import torch

    from sparse_long_sequence_longformer_amd import binding

    E, F = 64 * wl.H, args.ffn
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(11)
    x = torch.from_numpy(rng.standard_normal((wl.B, wl.L, E), dtype=np.float32)).to(torch.bfloat16).to(dev)
    shapes = {"w_qkv": (3 * E, E), "b_qkv": (3 * E,), "w_o": (E, E), "b_o": (E,), "ln1_g": (E,), "ln1_b": (E,),
              "w_1": (F, E), "b_1": (F,), "w_2": (E, F), "b_2": (E,), "ln2_g": (E,), "ln2_b": (E,)}
    W = {k: (torch.from_numpy(rng.standard_normal(sh, dtype=np.float32) * 0.05) + (1.0 if k.endswith("_g") else 0.0))
         .to(torch.bfloat16).to(dev) for k, sh in shapes.items()}
    out = binding.layer_forward(x, W, wl.w, dil, G, padd, handle=handle, causal=args.causal)
    torch.cuda.synchronize()
    lib = binding.load_library()
    i32p = ctypes.POINTER(ctypes.c_int32)
    dil_arr = (ctypes.c_int32 * len(dil))(*dil)
    g_arr = (ctypes.c_int32 * max(1, len(G)))(*G)
    wts = binding.LayerWeights(*[W[n].data_ptr() for n in binding.LAYER_WEIGHTS])
    args_c = (handle.handle, x.data_ptr(), ctypes.byref(wts), out.data_ptr(), wl.B, wl.L, E, F, ctypes.c_float(1e-5),
              wl.w, ctypes.cast(dil_arr, i32p), ctypes.cast(g_arr, i32p), len(G),
              None if padd is None else padd.data_ptr(), torch.cuda.current_stream().cuda_stream)

    def step():
        if lib.lf_layer_forward(*args_c) != 0:
            raise RuntimeError(lib.lf_attn_last_error(handle.handle).decode())

    clock = clock_warmup(step, args.clock_warmup, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    handle.set_stage_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    st = handle.stage_times()
    handle.set_stage_timing(False)
    per_call = {k2: v2[0] / args.steps for k2, v2 in st.items() if v2[1]}
    R = wl.B * wl.L
    gemm_flops = 2.0 * R * (3 * E * E + E * E + 2 * E * F)
    total = gemm_flops + flops_attn
    res = {
        "metric": "Longformer layer fwd effective TFLOP/s (GEMMs + window+global attention), L=4096 w=512",
        "value": round(total / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "clock_warmup_s": clock[0],
        "clock_warmup_steps": clock[1], "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0, 0.05^2) weights)",
        "config": {"workload": name, "B": wl.B, "seq_len": wl.L, "hidden": E, "heads": wl.H, "ffn": F, "w": wl.w,
                   "n_global": len(G), "parallelism": "single GPU",
                   "window": "one-sided" if args.causal else "symmetric",
                   "position_bias": f"N(0, {args.bias:g}^2) table" if args.bias else None,
                   "random_blocks": f"{args.random} of 64 keys per (head, query block)" if args.random else None},
        "tokens_per_s": round(R / (ms * 1e-3), 1),
        "gemm_flop": gemm_flops, "attention_flop": flops_attn,
        "stage_ms_per_layer": {k2: round(v2, 6) for k2, v2 in per_call.items()},
        "gemm_tflops": round(gemm_flops / (per_call.get("layer_gemm", float("nan")) * 1e-3) / 1e12, 3),
    }
    print(json.dumps(res), flush=True)


def bench_backward(args, wl, name, qd, kd, vd, padd, G, dil, pairs, flops_fwd, handle, gp=None):
    """Backward alone (inputs, forward output and log-sum-exp resident), then a whole
    training step (forward with log-sum-exp + backward).  Effective FLOP: 2.5 x the
    forward's (five products per attended pair instead of two).  gp: the separate
    projections (q_g, k_g, v_g) of the global rows, or None."""
    import numpy as np
    import torch

    from sparse_long_sequence_longformer_amd import binding

    g = np.random.default_rng(7).standard_normal(tuple(qd.shape), dtype=np.float32)
    dod = torch.from_numpy(g).to(torch.bfloat16).to(qd.device)
    if gp is None:
        out, lse = binding.forward_lse(qd, kd, vd, wl.w, dil, G, padd, handle=handle, causal=args.causal)
        grads = binding.backward(qd, kd, vd, out, dod, lse, wl.w, dil, G, padd, handle=handle, causal=args.causal)
    else:
        out, lse = binding.forward_global_proj_lse(qd, kd, vd, *gp, wl.w, dil, G, padd, handle=handle,
                                                   causal=args.causal)
        grads = binding.backward_global_proj(qd, kd, vd, *gp, out, dod, lse, wl.w, dil, G, padd, handle=handle,
                                             causal=args.causal)
    torch.cuda.synchronize()

    # The timed loops call the C entry points with arguments marshalled once: the
    # backward's four launches take less host time than the Python wrapper's checks.
    import ctypes

    lib = binding.load_library()
    i32p = ctypes.POINTER(ctypes.c_int32)
    dil_arr = (ctypes.c_int32 * len(dil))(*dil)
    g_arr = (ctypes.c_int32 * max(1, len(G)))(*G)
    stream = torch.cuda.current_stream().cuda_stream
    pad_ptr = None if padd is None else padd.data_ptr()
    shape = (wl.B, wl.H, wl.L, wl.d, wl.w, ctypes.cast(dil_arr, i32p), ctypes.cast(g_arr, i32p), len(G), pad_ptr,
             stream)
    qkv = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr())
    gptr = () if gp is None else tuple(t.data_ptr() for t in gp)
    bwd_args = (handle.handle, *qkv, *gptr, out.data_ptr(), dod.data_ptr(), lse.data_ptr(),
                *(t.data_ptr() for t in grads)) + shape
    fwd_args = (handle.handle, *qkv, *gptr, out.data_ptr(), lse.data_ptr()) + shape
    bwd_fn = lib.lf_attn_backward if gp is None else lib.lf_attn_backward_global_proj
    fwd_fn = lib.lf_attn_forward_lse if gp is None else lib.lf_attn_forward_global_proj_lse

    def bwd():
        if bwd_fn(*bwd_args) != 0:
            raise RuntimeError(lib.lf_attn_last_error(handle.handle).decode())

    def train_step():
        if fwd_fn(*fwd_args) != 0:
            raise RuntimeError(lib.lf_attn_last_error(handle.handle).decode())
        bwd()

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    clock = clock_warmup(bwd, args.clock_warmup, torch)
    for _ in range(args.warmup):
        bwd()
    torch.cuda.synchronize()
    ms_bwd = timed(bwd, args.steps)
    ms_train = timed(train_step, args.steps)
    handle.set_stage_timing(True)
    for _ in range(args.steps):
        bwd()
    torch.cuda.synchronize()
    st = handle.stage_times()
    handle.set_stage_timing(False)
    stage_avg = {k2: v2[0] / v2[1] for k2, v2 in st.items() if v2[1]}
    flops_bwd = 2.5 * flops_fwd
    # Products per attended pair: bwd_dq 3 (S, dP, dQ), bwd_dkv 4 (S, dP, dV, dK).
    per_pair = {"bwd_dq": 3 * 2 * wl.d, "bwd_dkv": 4 * 2 * wl.d}
    dom = max(per_pair, key=lambda k2: stage_avg.get(k2, 0.0))
    achieved = per_pair[dom] * pairs.total / (stage_avg[dom] * 1e-3) / 1e12
    value = flops_bwd / (ms_bwd * 1e-3) / 1e12
    res = {
        "metric": "window+global attn bwd effective TFLOP/s (2.5x forward FLOP), L=4096 w=512",
        "attended_pairs": pairs.total,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_warmup_s": clock[0],
        "clock_warmup_steps": clock[1],
        "ms_per_step": round(ms_bwd, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v/dO, no trained weights)",
        "config": {"workload": name, "B": wl.B, "H": wl.H, "seq_len": wl.L, "d_h": wl.d, "w": wl.w,
                   "dil": sorted(set(dil)), "n_global": len(G), "padded_lengths": list(wl.lengths) or None,
                   "global_batch": wl.B, "parallelism": "single GPU",
                   "window": "one-sided" if args.causal else "symmetric",
                   "position_bias": f"N(0, {args.bias:g}^2) table" if args.bias else None,
                   "random_blocks": f"{args.random} of 64 keys per (head, query block)" if args.random else None,
                   "global_projections": "separate" if gp is not None else "shared"},
        "pct_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 3),
        "train_step_ms": round(ms_train, 6),
        "train_step_tflops": round(3.5 * flops_fwd / (ms_train * 1e-3) / 1e12, 3),
        "kernel_ms_avg": {k2: round(v2, 6) for k2, v2 in stage_avg.items()},
        "roofline": {
            "kernel": f"lf::{dom}_kernel",
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "avg_launch_ms": round(stage_avg[dom], 6),
            "flop_per_launch": per_pair[dom] * pairs.total,
        },
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
