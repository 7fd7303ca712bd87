"""Phase timestamps of the single-launch 1-token layer step (diagnostic).

Loads libmoe_decode_phase.so (built by `python -m sparse_moe_decode_gemv_amd.build
--phase-trace`), runs the flagship layer (d=2048, f=512, E=256, top-8, int4)
over a pool of seeded layers -- isolated steps, then a pre-normed stack with one
launch per layer, each as a graph of consecutive launches -- and prints, for
every marked point of the last step of a replay, the minimum, median and
maximum over the workgroups, in microseconds from the first workgroup's
start, each the median over the replays.

    python -m sparse_moe_decode_gemv_amd.phase_trace [--pool 49] [--replays 12]
"""
from __future__ import annotations

import argparse
import os
import sys

PHASES = [
    "start (arguments read)",
    "x (or the normalized residual) in LDS",
    "router logits stored (router workgroups)",
    "every wave has the logits",
    "top-16 known in every wave",
    "this wave's gate/up loads issued",
    "selection done (barrier)",
    "gate/up and SwiGLU done",
    "h published",
    "all h in LDS",
    "end (down rows stored)",
]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--pool", type=int, default=49)
    ap.add_argument("--steps", type=int, default=64, help="launches per graph")
    ap.add_argument("--replays", type=int, default=12)
    ap.add_argument("--seed", type=int, default=1)
    args = ap.parse_args()

    import numpy as np
    import torch

    here = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, os.path.dirname(here))
    import synth
    import sparse_moe_decode_gemv_amd as M
    from sparse_moe_decode_gemv_amd import build as B

    if not os.path.exists(B.PHASE_LIB):
        raise RuntimeError(f"{B.PHASE_LIB} not built; run `python -m sparse_moe_decode_gemv_amd.build --phase-trace`")
    M.LIB_PATH = B.PHASE_LIB
    M.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.LAYER
    d, f, E, k = cfg.d, cfg.f, cfg.E, cfg.k
    P = args.pool
    layers = [M.MoELayer.create(M.upload(synth.make_layer(cfg, args.seed, l), dev), d, f, E, k, 1, 1) for l in range(P)]
    X = torch.from_numpy(np.stack([synth.draw_x(synth.STACK, args.seed, l, 0, 0) for l in range(P)]).view(np.int16)).to(dev)
    y = torch.empty((1, d), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    buf = np.zeros(1024 * 16, np.uint64)
    G = torch.cuda.get_device_properties(dev).multi_processor_count
    n_router = (E + 3) // 4

    def read():
        torch.cuda.synchronize()
        M.moe_decode_phase_trace(buf)
        t = buf.reshape(1024, 16)[:G, :len(PHASES)].astype(np.int64)
        return (t - t[:, 0].min()) * 10 / 1000.0  # 100 MHz counter -> us

    def run(name, step, per_launch):
        with torch.cuda.stream(s):
            step(0)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(args.steps):
                step(i)
        runs = []
        for _ in range(args.replays):
            g.replay()
            runs.append(read())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record(s)
            g.replay()
            e1.record(s)
        e1.synchronize()
        a = np.stack(runs)  # [replays][workgroups][phases]
        print(f"{name}: {e0.elapsed_time(e1) * 1e3 / (args.steps * per_launch):.3f} us per launch in the graph")
        print("  phase                                        min      median   max   (us; median of replays)")
        for ph, label in enumerate(PHASES):
            v = a[:, :n_router, ph] if ph == 2 else a[:, :, ph]
            print(f"  {ph:2d} {label:40s} {np.median(v.min(1)):7.2f} {np.median(np.median(v, 1)):8.2f} "
                  f"{np.median(v.max(1)):7.2f}")

    run(f"isolated steps ({P} layers rotated, x from the caller)",
        lambda i: M.moe_decode_forward(layers[i % P].handle, X[i % P:i % P + 1], 1, y, None, None, s), 1)

    base = torch.from_numpy(synth.draw_x(synth.STACK, args.seed, 0, 0, 0).view(np.int16)[None]).view(
        torch.bfloat16).float().to(dev)
    resid = torch.empty((1, d), dtype=torch.float32, device=dev)
    hs = [L.handle for L in layers]

    def sstep(i):
        resid.copy_(base)
        M.moe_decode_stack_forward(hs, resid, 1, 1e-6, None, None, None, s)

    args.steps = 4
    run(f"{P}-layer stack, one launch per layer (the last layer's phases)", sstep, P)


if __name__ == "__main__":
    main()
