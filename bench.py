"""Benchmark: MoE-layer decode tokens/s at 1 token + achieved HBM GB/s.

Workload (one step = one token through one MoE layer: router GEMV, softmax
and top-k, int4 gate/up GEMVs over the 8 chosen experts, SwiGLU, int4 down
GEMV and weighted combine): d=2048, f=512, E=256, top-8, int4 weights with
one fp16 scale per 32, bf16 activations.  The pages give no layer shapes;
these reproduce their totals (256 routed experts per layer, 40B total, 2.5B
active, "Flint 40B: Best Mid Sized LLM", transcript 02:35).

So that the 256 MB memory-side cache cannot serve repeats, steps rotate over
a pool of P = 49 independent seeded layers (22.3 GB of weights, the 49-layer
stack's layers) with a fresh activation, and every timed window of K steps
(eager launches; window r starts at layer r*K mod P) follows a 1 GiB read:
every step reads its router and chosen experts from HBM, whatever K is.  The same windows as one HIP-graph replay each are reported beside it
(a replay carries a fixed cost of tens of microseconds).

Also reported (not the headline): the 49-layer stack per-token time, the
LM head (V=131072, d=2048) at B=1 and B=8, and the plain fp64 CPU oracle
timed on a bounded sample of the same workload.

Prints one JSON line.  `--gpus N` with N > 1 exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
KERNEL_SOURCES = ["sparse_moe_decode_gemv_amd/csrc/layer_kernel.h", "sparse_moe_decode_gemv_amd/csrc/kernels_layer.hip",
                  "sparse_moe_decode_gemv_amd/csrc/device_common.h", "sparse_moe_decode_gemv_amd/csrc/topk.h"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def layer_bytes(d, f, E, k):
    """Algorithmic bytes of one 1-token layer step: router weights, x, the k
    chosen experts' int4 nibbles + fp16 scales (each read once), y."""
    nib = k * (2 * f * d // 2 + d * f // 2)
    scales = k * (2 * f * (d // 32) * 2 + d * (f // 32) * 2)
    router = E * d * 4
    return dict(b_nib=nib, b_q=nib + scales, b_alg=nib + scales + router + d * 2 + d * 4)


def lmhead_bytes(V, d, B):
    return V * d // 2 + V * (d // 32) * 2 + B * d * 2 + B * 8


def time_graph(fn, steps, warmup, stream, warm_s=0.0):
    """Capture `fn(i)` for i in range(steps) into one graph; return seconds per replay.
    warm_s: keep replaying for at least this long before timing (a leg that
    follows seconds of host-side setup otherwise starts on an idle GPU)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for i in range(min(warmup, steps)):
            fn(i)
    stream.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            fn(i)
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.time()
    while time.time() - t0 < warm_s:
        g.replay()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    reps = 3
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(reps):
            g.replay()
        end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / 1e3 / reps, g


def time_launches(fn, steps, stream):
    """Mean duration of the launch each `fn(i)` enqueues, from hipEventRecord
    pairs on `stream` around every launch.  A few ms of fills are queued
    first, so that every pair is enqueued before the GPU reaches it and no
    host gap falls inside a pair (the gaps between pairs are reported)."""
    import ctypes

    import torch
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch has loaded
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = [ctypes.c_void_p() for _ in range(2 * steps)]
    for e in evs:
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
    sh = ctypes.c_void_p(stream.cuda_stream)
    pad = torch.empty(256 << 20, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(stream):
        for _ in range(48):
            pad.fill_(1.0)
        for i in range(steps):
            hip.hipEventRecord(evs[2 * i], sh)
            fn(i)
            hip.hipEventRecord(evs[2 * i + 1], sh)
    stream.synchronize()
    ms = ctypes.c_float()

    def el(a, b):
        if hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e3

    ts = sorted(el(evs[2 * i], evs[2 * i + 1]) for i in range(steps))
    gaps = sorted(el(evs[2 * i + 1], evs[2 * i + 2]) for i in range(steps - 1))
    for e in evs:
        hip.hipEventDestroy(e)
    del pad
    return dict(mean_us=sum(ts) / len(ts), median_us=ts[len(ts) // 2], p10_us=ts[len(ts) // 10],
                p90_us=ts[len(ts) * 9 // 10], median_gap_us=gaps[len(gaps) // 2] if gaps else 0.0)


def traffic_from_profile(kernel_sources, name):
    """HBM bytes per launch measured with rocprofv3 counters and recorded in
    profiles/<name>; None unless the recorded source hash matches the kernel
    sources as they are now."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for src in kernel_sources:
        with open(os.path.join(ROOT, src), "rb") as fh:
            h.update(fh.read())
    rec = {}
    with open(path) as fh:
        for ln in fh:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("sources_sha256") != h.hexdigest():
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_eager(fn, steps, warmup, stream):
    import torch
    with torch.cuda.stream(stream):
        for i in range(warmup):
            fn(i)
        stream.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(steps):
            fn(i)
        end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / 1e3


def cpu_baseline(pool_np, xs_np, cfg, steps_per_run, runs=5):
    """The plain C++ fp64 oracle as it stands, on a bounded sample of the same
    steps: `runs` timed runs of `steps_per_run` single-token layer steps,
    once single-threaded and once with OpenMP over the threads the process
    may use (OMP_NUM_THREADS, else every hardware thread); medians.  The
    numpy fp64 oracle is timed the same way beside it, with one BLAS thread
    and with the default pool."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import cpp_oracle as CO
    from oracle import moe as OM

    layers = [CO.CLayer(p) for p in pool_np]

    def run_cpp():
        t0 = time.perf_counter()
        for n in range(steps_per_run):
            li = n % len(layers)
            CO.moe_forward(layers[li], xs_np[li][n % len(xs_np[li])], cfg.k)
        return time.perf_counter() - t0

    def run_numpy():
        t0 = time.perf_counter()
        for n in range(steps_per_run):
            li = n % len(pool_np)
            OM.moe_forward(OM.Layer.from_dict(pool_np[li]), xs_np[li][n % len(xs_np[li])], cfg.k)
        return time.perf_counter() - t0

    n_omp = CO.get_threads()
    run_cpp()  # first touch of the layers' pages
    CO.set_threads(1)
    single = sorted(run_cpp() for _ in range(runs))
    CO.set_threads(n_omp)
    multi = sorted(run_cpp() for _ in range(runs))
    with threadpool_limits(1):
        np1 = sorted(run_numpy() for _ in range(runs))
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    npn = sorted(run_numpy() for _ in range(runs))
    med = lambda v: v[runs // 2]  # noqa: E731
    rate = lambda t: round(steps_per_run / t, 3)  # noqa: E731
    nl = min(steps_per_run, len(pool_np))
    return dict(value=rate(med(multi)), unit="tokens/s", cores=n_omp, kind="oracle",
                host_cores=CO.hw_threads(),
                single_thread={"value": rate(med(single)), "unit": "tokens/s", "cores": 1},
                numpy_oracle={"value": rate(med(npn)), "cores": blas, "single_thread": rate(med(np1)),
                              "unit": "tokens/s"},
                sample=f"{runs} runs of {steps_per_run} single-token layer steps over {nl} layers of the pool, "
                       f"median; plain C++ fp64 oracle with OpenMP over {n_omp} threads (value) and single-threaded "
                       f"(single_thread); host hardware threads {CO.hw_threads()}; the numpy fp64 oracle beside it")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=490)
    ap.add_argument("--warmup", type=int, default=49)
    ap.add_argument("--pool", type=int, default=49, help="distinct layers rotated through")
    ap.add_argument("--tokens", type=int, default=16, help="distinct activations per layer")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-steps", type=int, default=8, help="oracle steps per timed run (5 runs per thread setting)")
    ap.add_argument("--no-extras", action="store_true", help="skip stack, batch, LM head and CPU legs")
    ap.add_argument("--extras", default="stack,batch,prefill,flint,fp4,lmhead,cpu",
                    help="comma list of the legs run after the headline (stack, batch, prefill, flint, fp4, lmhead, cpu)")
    ap.add_argument("--windows", type=int, default=7, help="timed windows of K steps (median reported)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import sparse_moe_decode_gemv_amd as M

    M.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return
    cfg = synth.LAYER
    d, f, E, k = cfg.d, cfg.f, cfg.E, cfg.k
    P = args.pool

    t0 = time.time()
    layers, pool_np, xs_np = [], [], []
    keep_host = 2  # host copies kept for the CPU leg
    for l in range(P):
        lay = synth.make_layer(cfg, args.seed, l)
        layers.append(M.MoELayer.create(M.upload(lay, dev), d, f, E, k, 1, 1))
        xs = np.stack([synth.draw_x(synth.STACK, args.seed, l, t, 0) for t in range(args.tokens)])
        xs_np.append(xs)
        if l < keep_host:
            pool_np.append(lay)
        del lay
    X = torch.from_numpy(np.stack(xs_np).view(np.int16)).to(dev)  # [P][tokens][d]
    torch.cuda.synchronize()
    log(f"pool of {P} layers generated and uploaded in {time.time() - t0:.1f} s")

    y = torch.empty((1, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    # Reading 1 GiB (four times the 256 MB memory-side cache) leaves it full
    # of clean lines of another buffer; a write would leave dirty lines whose
    # write-back the next steps would pay for.
    flush = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
    flush_sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def mall_flush():
        M.moe_decode_read_probe(flush, flush.numel(), flush_sink, stream)

    def step_at(off):
        def step(i):
            j = off + i
            l = j % P
            t = (j // P) % args.tokens
            M.moe_decode_forward(layers[l].handle, X[l, t:t + 1], 1, y, None, None, stream)
        return step

    step = step_at(0)
    K, W = args.steps, args.warmup
    eager_s = time_eager(step, K, W, stream)

    # A GPU-side pause after the write, long enough for the host to enqueue
    # a whole window (about 10 us of Python per launch), so that the timed
    # region holds GPU time only: torch's spin kernel, its cycles calibrated
    # against events once.
    with torch.cuda.stream(stream):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.cuda._sleep(1 << 20)
        e1.record(stream)
    e1.synchronize()
    cycles_per_us = (1 << 20) / max(e0.elapsed_time(e1) * 1e3, 1.0)

    def windows(launch_window):
        """Per-step times of args.windows timed windows of exactly K steps,
        each after a 1 GiB read and a pause covering the host's enqueue;
        window r starts at layer r*K mod P."""
        out_us = []
        for r in range(args.windows):
            mall_flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                torch.cuda._sleep(int(cycles_per_us * (200 + 25 * K)))
                e0.record(stream)
                launch_window(r)
                e1.record(stream)
            e1.synchronize()
            out_us.append(e0.elapsed_time(e1) * 1e3 / K)
        return out_us

    win_us = windows(lambda r: [step_at(r * K)(i) for i in range(K)])
    gwin_us = []
    try:  # the same windows as K-node graph replays (one replay per window)
        ng = max(1, min(4, (P + K - 1) // K))
        graphs = []
        for j in range(ng):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(K):
                    step_at(j * K)(i)
            graphs.append(g)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        gwin_us = windows(lambda r: graphs[r % ng].replay())
        del graphs
    except Exception as e:  # graph capture unavailable
        log(f"graph capture failed: {e!r}")
    win_s = sorted(win_us)[len(win_us) // 2] * K / 1e6
    graph_s = sorted(gwin_us)[len(gwin_us) // 2] * K / 1e6 if gwin_us else None
    total_s = win_s
    ms_per_step = total_s / K * 1e3
    value = K / total_s

    by = layer_bytes(d, f, E, k)
    step_us = ms_per_step * 1e3
    try:
        kt = time_launches(step, min(K, 196), stream)
    except Exception as e:  # noqa: BLE001
        log(f"event-pair timing failed: {e!r}")
        kt = None
    # The step is one launch of one kernel, so the launch duration is the
    # step time between the HIP events bracketing the timed region on the
    # launch stream (it agrees with the kernel-trace average).  Event pairs
    # around single launches add the markers' own cost; reported aside.
    kernel_us = step_us
    achieved = by["b_alg"] / (kernel_us * 1e-6) / 1e9

    # Cold single calls: each after a 1 GiB write, so that neither the
    # memory-side cache nor the L2 holds anything of the layer; events around
    # one eager call, enqueued while the write runs.
    cold = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold_us = []
    for r in range(5):
        with torch.cuda.stream(stream):
            cold.fill_(r)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step(7 * r + 3)
            e1.record(stream)
        e1.synchronize()
        cold_us.append(e0.elapsed_time(e1) * 1e3)
    cold_us.sort()
    # Achievable read bandwidth: the library's plain streaming read of a
    # 2 GiB buffer, after the 1 GiB write (so the memory-side cache holds
    # none of it); median of 5.
    probe = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    probe_us = []
    for r in range(6):
        with torch.cuda.stream(stream):
            cold.fill_(r)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            M.moe_decode_read_probe(probe, probe.numel(), sink, stream)
            e1.record(stream)
        e1.synchronize()
        if r:
            probe_us.append(e0.elapsed_time(e1) * 1e3)
    probe_us.sort()
    achievable = probe.numel() / (probe_us[len(probe_us) // 2] * 1e-6) / 1e9
    del probe, cold
    wins = sorted(win_us) if win_us else [step_us]
    out = {
        "metric": "MoE-layer decode tokens/s at 1 token + achieved HBM GB/s (% of peak)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4-bf16-f32",
        "data": "synthetic (seeded N(0,0.02) int4 g32 fp16-scale experts, fp32 router, bf16 N(0,1) x)",
        "config": {"workload": "1-token MoE layer decode, d=2048 f=512 E=256 top-8, "
                               f"rotating over {P} distinct layers, fresh x per step",
                   "d": d, "f": f, "experts": E, "top_k": k, "tokens_per_step": 1, "pool_layers": P,
                   "launch": "eager launches, timed in windows of K steps after a 1 GiB read"},
        "roofline": {"bound": "hbm", "kernel": "k_layer (whole 1-token layer step, one launch)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_from_profile(KERNEL_SOURCES, "traffic_k_layer_flagship.txt"),
                     "bytes_per_launch": by["b_alg"],
                     "launch_us": round(kernel_us, 3),
                     "launch_timing": "HIP events around each timed window of K steps on the launch stream / "
                                      "K (one launch per step); median window",
                     "achievable": round(achievable, 1),
                     "frac_of_achievable": round(achieved / achievable, 4)},
        "step_us": {"median": round(step_us, 3), "p10": round(wins[len(wins) // 10], 3),
                    "p90": round(wins[(len(wins) * 9) // 10], 3), "windows": len(win_us),
                    "over": "per-step time of each timed window of K steps (each after a 1 GiB read)"},
        "launch_event_pairs_us": ({k2: round(v, 3) for k2, v in kt.items()} if kt else None),
        "cold_call_us": {"median": round(cold_us[len(cold_us) // 2], 3), "min": round(cold_us[0], 3),
                         "max": round(cold_us[-1], 3), "calls": len(cold_us),
                         "over": "one eager call after a 1 GiB write, HIP events around it"},
        "read_probe": {"gbs": round(achievable, 1), "bytes": 2 << 30, "frac_of_peak": round(achievable / PEAK_HBM_GBS, 4),
                       "us": round(probe_us[len(probe_us) // 2], 2)},
        "bytes_per_step": by,
        "gbs_on_int4_weights": round(by["b_q"] / (step_us * 1e-6) / 1e9, 1),
        "frac_on_int4_weights": round(by["b_q"] / (step_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "eager_ms_per_step": round(eager_s / K * 1e3, 6),
        "graph_window_ms_per_step": round(graph_s / K * 1e3, 6) if graph_s else None,
    }

    extras = set() if args.no_extras else {e.strip() for e in args.extras.split(",") if e.strip()}
    if "stack" in extras:
        # 49-layer stack, 1 token: per-token time (in-stack layer time = / P)
        # r_0 = fp32 of a bf16 N(0,1) activation, as in the stack's definition
        x0 = synth.draw_x(synth.STACK, args.seed, 0, 0, 0)
        base = torch.from_numpy(x0.view(np.int16)[None]).view(torch.bfloat16).float().to(dev)
        resid = torch.empty((1, d), dtype=torch.float32, device=dev)
        handles = [L.handle for L in layers]

        def stack_time(flags):
            def stack_step(i):
                resid.copy_(base)
                M.moe_decode_stack_forward_ex(handles, resid, 1, 1e-6, None, None, None, flags, stream)

            st_s = time_eager(stack_step, 10, 2, stream) / 10
            try:
                gs, _g = time_graph(stack_step, 10, 2, stream)
                st_s = gs / 10
                del _g
            except Exception as e:
                log(f"stack graph failed: {e!r}")
            return st_s

        st_s = stack_time(0)
        sp_s = stack_time(M.MOE_STACK_PERSISTENT)
        out["stack"] = {"layers": P, "ms_per_token": round(st_s * 1e3, 4),
                        "tokens_per_s": round(1 / st_s, 1),
                        "in_stack_layer_us": round(st_s / P * 1e6, 3),
                        "achieved_gbs": round(P * by["b_alg"] / st_s / 1e9, 1),
                        "launch": "one launch per layer, graph"}
        out["stack_persistent"] = {"layers": P, "ms_per_token": round(sp_s * 1e3, 4),
                                   "tokens_per_s": round(1 / sp_s, 1),
                                   "in_stack_layer_us": round(sp_s / P * 1e6, 3),
                                   "achieved_gbs": round(P * by["b_alg"] / sp_s / 1e9, 1),
                                   "launch": "one persistent launch for the 49 layers (MOE_STACK_PERSISTENT), graph"}

    if "batch" in extras:
        # batch: 64 tokens per call through one layer, Zipf(1.1) router bias
        TB = synth.BATCH.T
        bias = torch.from_numpy(synth.zipf_bias(synth.BATCH, args.seed)).to(dev)
        blayers = [M.MoELayer.create(dict(L.tensors, router_b=bias), d, f, E, k, 1, TB) for L in layers]
        XB = torch.from_numpy(np.stack([np.stack([synth.draw_x(synth.BATCH, args.seed, l, t, 0) for t in range(TB)])
                                        for l in range(P)]).view(np.int16)).to(dev)  # [P][TB][d]
        yb = torch.empty((TB, d), dtype=torch.float32, device=dev)
        ib = torch.empty((P, TB, k), dtype=torch.int32, device=dev)
        for l in range(P):
            M.moe_decode_forward(blayers[l].handle, XB[l], TB, yb, ib[l], None, stream)
        stream.synchronize()
        distinct = [len(np.unique(a)) for a in ib.cpu().numpy()]

        def batch_step(i):
            l = i % P
            M.moe_decode_forward(blayers[l].handle, XB[l], TB, yb, None, None, stream)

        nb = 2 * P
        try:
            bs, _g = time_graph(batch_step, nb, P, stream)
            del _g
        except Exception as e:
            log(f"batch graph failed: {e!r}")
            bs = time_eager(batch_step, nb, P, stream)
        us = bs / nb * 1e6
        per_expert = by["b_q"] // k
        b_batch = E * d * 4 + TB * d * 2 + float(np.mean(distinct)) * per_expert + TB * d * 4
        out["batch_t64"] = {"us_per_call": round(us, 3), "tokens_per_s": round(TB / (us * 1e-6), 1),
                            "distinct_experts_mean": round(float(np.mean(distinct)), 2),
                            "distinct_experts_range": [int(min(distinct)), int(max(distinct))],
                            "bytes_per_call": int(b_batch), "achieved_gbs": round(b_batch / (us * 1e-6) / 1e9, 1),
                            "frac": round(b_batch / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        for L in blayers:
            L.close()
        del blayers, XB

    if "prefill" in extras:
        # prompt processing: 2048 tokens per call through one layer (no
        # router bias), rotating over 8 layers of the pool (4.7 GB with their
        # tile-major copies, more than the memory-side cache)
        TP, PL = 2048, 8
        pl = [M.MoELayer.create(layers[l].tensors, d, f, E, k, 1, TP) for l in range(PL)]
        XP = torch.from_numpy(np.stack([np.stack([synth.draw_x(synth.LAYER, args.seed, l, 4096 + t, 0)
                                                  for t in range(TP)]) for l in range(PL)]).view(np.int16)).to(dev)
        yp = torch.empty((TP, d), dtype=torch.float32, device=dev)
        ipf = torch.empty((PL, TP, k), dtype=torch.int32, device=dev)
        for l in range(PL):
            M.moe_decode_forward(pl[l].handle, XP[l], TP, yp, ipf[l], None, stream)
        stream.synchronize()
        dpf = [len(np.unique(a)) for a in ipf.cpu().numpy()]

        def prefill_step(i):
            M.moe_decode_forward(pl[i % PL].handle, XP[i % PL], TP, yp, None, None, stream)

        try:
            ps, _g = time_graph(prefill_step, 4 * PL, PL, stream)
            del _g
        except Exception as e:
            log(f"prefill graph failed: {e!r}")
            ps = time_eager(prefill_step, 4 * PL, PL, stream)
        us = ps / (4 * PL) * 1e6
        per_expert = by["b_q"] // k
        bp = E * d * 4 + TP * d * 2 + float(np.mean(dpf)) * per_expert + TP * d * 4
        flop = TP * (2 * E * d + k * 3 * 2 * d * f)
        out["prefill_t2048"] = {"us_per_call": round(us, 3), "tokens_per_s": round(TP / (us * 1e-6), 1),
                                "distinct_experts_mean": round(float(np.mean(dpf)), 2),
                                "bytes_per_call": int(bp), "achieved_gbs": round(bp / (us * 1e-6) / 1e9, 1),
                                "frac": round(bp / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                                "tflops": round(flop / (us * 1e-6) / 1e12, 1)}
        for L in pl:
            L.close()
        del pl, XP

    if "flint" in extras:
        # the pages' own routing: top-6 of the 256 routed experts plus one
        # shared expert, 1-token steps over the same pool (each layer gets its
        # shared expert), graph-timed like the headline
        fk = synth.FLINT.k
        fl = []
        for l, L in enumerate(layers):
            sh = M.upload(synth.make_shared(synth.FLINT, args.seed, l), dev)
            fl.append(M.MoELayer.create(dict(L.tensors, **sh), d, f, E, fk, 1, 1))
        yf = torch.empty((1, d), dtype=torch.float32, device=dev)

        def flint_step(i):
            l = i % P
            t = (i // P) % args.tokens
            M.moe_decode_forward(fl[l].handle, X[l, t:t + 1], 1, yf, None, None, stream)

        try:
            fs, _g = time_graph(flint_step, 2 * P * 5, P, stream)
            del _g
        except Exception as e:
            log(f"flint graph failed: {e!r}")
            fs = time_eager(flint_step, 2 * P * 5, P, stream)
        us = fs / (2 * P * 5) * 1e6
        bf = E * d * 4 + d * 2 + (fk + 1) * (by["b_q"] // k) + d * 4
        out["flint_top6_shared"] = {"us_per_step": round(us, 3), "tokens_per_s": round(1 / (us * 1e-6), 1),
                                    "bytes_per_step": int(bf), "achieved_gbs": round(bf / (us * 1e-6) / 1e9, 1),
                                    "frac": round(bf / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        for L in fl:
            L.close()
        del fl

    if "fp4" in extras:
        # FP4 experts, MXFP4 (E2M1 codes, E8M0 scale per 32) and NVFP4 (E4M3
        # scale per 16 + fp32 per matrix): the same draws as the pool's first
        # 16 layers quantized to FP4 (6.7 GB, beyond the memory-side cache);
        # 1-token steps graph-timed like the headline, then the batched call
        # at T = 64 with the Zipf bias on the same layers
        PF = min(16, P)
        TB = synth.BATCH.T
        bias = torch.from_numpy(synth.zipf_bias(synth.BATCH, args.seed)).to(dev)
        XB4 = torch.from_numpy(np.stack([np.stack([synth.draw_x(synth.BATCH, args.seed, l, t, 0) for t in range(TB)])
                                         for l in range(PF)]).view(np.int16)).to(dev)
        for fname, fcfg, sbytes in (("mxfp4", synth.LAYER_FP4, 3 * f * (d // 32)),
                                    ("nvfp4", synth.LAYER_NV, 3 * f * (d // 16) + 12)):
            f4 = [M.MoELayer.create(M.upload(synth.make_layer(fcfg, args.seed, l), dev), d, f, E, k, 1, 1)
                  for l in range(PF)]
            y4 = torch.empty((1, d), dtype=torch.float32, device=dev)

            def fp4_step(i, f4=f4, y4=y4):
                l = i % PF
                t = (i // PF) % args.tokens
                M.moe_decode_forward(f4[l].handle, X[l, t:t + 1], 1, y4, None, None, stream)

            try:
                f4s, _g = time_graph(fp4_step, 30 * PF, PF, stream)
                del _g
            except Exception as e:
                log(f"{fname} graph failed: {e!r}")
                f4s = time_eager(fp4_step, 30 * PF, PF, stream)
            us = f4s / (30 * PF) * 1e6
            per_expert4 = 3 * f * d // 2 + sbytes  # codes + scales
            b4 = E * d * 4 + d * 2 + k * per_expert4 + d * 4
            out[f"{fname}_layer"] = {"us_per_step": round(us, 3), "tokens_per_s": round(1 / (us * 1e-6), 1),
                                     "bytes_per_step": int(b4), "achieved_gbs": round(b4 / (us * 1e-6) / 1e9, 1),
                                     "frac": round(b4 / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "pool_layers": PF}
            fb = [M.MoELayer.create(dict(L.tensors, router_b=bias), d, f, E, k, 1, TB) for L in f4]
            for L in f4:
                L.close()
            del f4
            yb4 = torch.empty((TB, d), dtype=torch.float32, device=dev)
            ib4 = torch.empty((PF, TB, k), dtype=torch.int32, device=dev)
            for l in range(PF):
                M.moe_decode_forward(fb[l].handle, XB4[l], TB, yb4, ib4[l], None, stream)
            stream.synchronize()
            d4 = [len(np.unique(a)) for a in ib4.cpu().numpy()]

            def fp4_batch_step(i, fb=fb, yb4=yb4):
                M.moe_decode_forward(fb[i % PF].handle, XB4[i % PF], TB, yb4, None, None, stream)

            try:
                f4b, _g = time_graph(fp4_batch_step, 4 * PF, PF, stream)
                del _g
            except Exception as e:
                log(f"{fname} batch graph failed: {e!r}")
                f4b = time_eager(fp4_batch_step, 4 * PF, PF, stream)
            us = f4b / (4 * PF) * 1e6
            b4b = E * d * 4 + TB * d * 2 + float(np.mean(d4)) * per_expert4 + TB * d * 4
            out[f"{fname}_batch_t64"] = {"us_per_call": round(us, 3), "tokens_per_s": round(TB / (us * 1e-6), 1),
                                         "distinct_experts_mean": round(float(np.mean(d4)), 2),
                                         "bytes_per_call": int(b4b), "achieved_gbs": round(b4b / (us * 1e-6) / 1e9, 1),
                                         "frac": round(b4b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            for L in fb:
                L.close()
            del fb
        del XB4

    if "lmhead" in extras:
        # LM head: rotate over 4 copies; 0.1 s of replays before timing (the
        # heads are generated on the host first, leaving the GPU idle)
        V = synth.LMHEAD1.V
        heads = []
        for c in range(4):
            q, s = synth.make_lmhead(synth.LMHEAD1, args.seed, c)
            heads.append((torch.from_numpy(q).to(dev), torch.from_numpy(s.view(np.int16)).to(dev)))
        del q, s
        for B in (1, 8):
            xb = torch.from_numpy(
                np.stack([synth.draw_hidden(synth.LMHEAD8, args.seed, b, 0) for b in range(B)]).view(np.int16)).to(dev)
            tok = torch.empty(B, dtype=torch.int32, device=dev)
            ml = torch.empty(B, dtype=torch.float32, device=dev)
            wsz = M.lmhead_int4_argmax_workspace_bytes(V, d, B)
            wsp = torch.zeros(wsz, dtype=torch.uint8, device=dev)

            def lm_step(i, B=B, xb=xb, tok=tok, ml=ml, wsp=wsp):
                wq, wsc = heads[i % 4]
                M.lmhead_int4_argmax(wq, wsc, V, d, xb, B, tok, ml, wsp, wsz, stream)

            n = 40
            try:
                ls, _g = time_graph(lm_step, n, 4, stream, warm_s=0.1)
                del _g
            except Exception as e:
                log(f"lmhead graph failed: {e!r}")
                ls = time_eager(lm_step, n, 4, stream)
            us = ls / n * 1e6
            gbs = lmhead_bytes(V, d, B) / (us * 1e-6) / 1e9
            out[f"lmhead_b{B}"] = {"us_per_call": round(us, 3), "rows_per_s": round(B / (us * 1e-6), 1),
                                   "achieved_gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
        del heads

    if "cpu" in extras:
        cb = cpu_baseline(pool_np, xs_np, cfg, args.cpu_steps)
        # the oracle's rate as algorithmic bytes per second, as for the GPU legs
        cb["gbs_on_b_alg"] = round(cb["value"] * by["b_alg"] / 1e9, 3)
        cb["single_thread"]["gbs_on_b_alg"] = round(cb["single_thread"]["value"] * by["b_alg"] / 1e9, 3)
        out["cpu_baseline"] = cb

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
