"""Parity in the launch configuration the benchmark times: the calls
captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.  Every replay,
with other eager work and synchronizations between replays, must give the
eager calls' outputs bit for bit (same kernels, same inputs, no hidden
state but the per-workgroup call counts), and sampled steps must match the
fp64 oracle.  Covers the 1-token steps over a pool of flagship layers with
fresh activations, the batched T=64 call, an odd-length pre-normed stack
(its final residual copy is a graph node) and the LM head at B=8."""
import numpy as np
import pytest

import synth
import sparse_moe_decode_gemv_amd as M
from gpu_common import Y_TOL, device, tokens
from oracle import formats as F
from oracle import moe as OM

pytestmark = pytest.mark.gpu


def capture(fn, n, stream):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def replay_checked(g, outs_eager, outs_graph, reps=3):
    """Replay g reps times; eager work and a sync between replays; every
    replay's outputs equal the eager ones bit for bit."""
    import torch
    for r in range(reps):
        for o in outs_graph:
            o.fill_(float("nan") if o.dtype.is_floating_point else -1)
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 16, device=outs_graph[0].device).sum()  # other eager work
        torch.cuda.synchronize()
        del junk
        for a, b in zip(outs_eager, outs_graph):
            if a.dtype.is_floating_point:  # bit patterns (NaN-safe)
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), f"replay {r} differs from eager"


def test_headline_steps_in_a_graph():
    """16 one-token steps over 8 flagship layers (layer i % 8, a fresh
    margin-conditioned token per step), as the benchmark runs them."""
    import torch
    dev = device()
    cfg = synth.LAYER
    P, S = 8, 16
    lays = [synth.make_layer(cfg, 1, l) for l in range(P)]
    OLs = [OM.Layer.from_dict(l) for l in lays]
    Ls = [M.MoELayer.create(M.upload(l, dev), cfg.d, cfg.f, cfg.E, cfg.k, 1, 1) for l in lays]
    X = np.stack([tokens(cfg, OLs[i % P], 1, 1, lidx=i % P)[0] for i in range(S)])
    Xd = torch.from_numpy(X.view(np.int16)).to(dev)
    stream = torch.cuda.Stream()

    def run(y, idx):
        def step(i):
            M.moe_decode_forward(Ls[i % P].handle, Xd[i:i + 1], 1, y[i:i + 1], idx[i:i + 1], None, stream)
        return step

    ye = torch.empty((S, cfg.d), dtype=torch.float32, device=dev)
    ie = torch.empty((S, cfg.k), dtype=torch.int32, device=dev)
    with torch.cuda.stream(stream):
        for i in range(S):
            run(ye, ie)(i)
    torch.cuda.synchronize()
    yg = torch.empty_like(ye)
    ig = torch.empty_like(ie)
    g = capture(run(yg, ig), S, stream)
    replay_checked(g, [ye, ie], [yg, ig])
    y, idx = ye.cpu().numpy(), ie.cpu().numpy()
    for i in (0, 5, 11, 15):
        out = OM.moe_forward_tokens(OLs[i % P], X[i:i + 1], cfg.k)
        assert np.array_equal(np.sort(idx[i]), np.sort(out["idx"][0])), f"step {i}: experts"
        err = np.abs(y[i].astype(np.float64) - out["y"][0]).max()
        assert err <= Y_TOL * np.abs(out["y"][0]).max(), f"step {i}: y err {err:.3e}"
    # every bounded wait of every replayed step completed
    for L in Ls:
        assert L.error_flags() == 0
        L.close()


def test_batched_call_in_a_graph():
    """The T=64 Zipf-biased call on two layers, captured and replayed."""
    import torch
    dev = device()
    cfg = synth.BATCH
    lays = [synth.make_layer(cfg, 2, l) for l in range(2)]
    OLs = [OM.Layer.from_dict(l) for l in lays]
    Ls = [M.MoELayer.create(M.upload(l, dev), cfg.d, cfg.f, cfg.E, cfg.k, 1, cfg.T) for l in lays]
    Xs = [tokens(cfg, OLs[l], 2, cfg.T, lidx=l) for l in range(2)]
    Xd = [torch.from_numpy(x.view(np.int16)).to(dev) for x in Xs]
    stream = torch.cuda.Stream()

    def run(y, idx):
        def step(i):
            M.moe_decode_forward(Ls[i].handle, Xd[i], cfg.T, y[i], idx[i], None, stream)
        return step

    ye = torch.empty((2, cfg.T, cfg.d), dtype=torch.float32, device=dev)
    ie = torch.empty((2, cfg.T, cfg.k), dtype=torch.int32, device=dev)
    with torch.cuda.stream(stream):
        for i in range(2):
            run(ye, ie)(i)
    torch.cuda.synchronize()
    yg, ig = torch.empty_like(ye), torch.empty_like(ie)
    g = capture(run(yg, ig), 2, stream)
    replay_checked(g, [ye, ie], [yg, ig])
    sample = [0, 17, 40, 63]
    for l in range(2):
        out = OM.moe_forward_tokens(OLs[l], Xs[l][sample], cfg.k)
        y, idx = ye[l].cpu().numpy()[sample], ie[l].cpu().numpy()[sample]
        for t in range(len(sample)):
            assert np.array_equal(np.sort(idx[t]), np.sort(out["idx"][t]))
            err = np.abs(y[t].astype(np.float64) - out["y"][t]).max()
            assert err <= Y_TOL * np.abs(out["y"][t]).max()
    for L in Ls:
        L.close()


def test_odd_stack_in_a_graph():
    """A 5-layer pre-normed stack at the flagship shape (odd: its last step
    is a residual copy), the residual reset inside the graph as the
    benchmark does."""
    import torch
    dev = device()
    cfg = synth.STACK
    lays = [synth.make_layer(cfg, 3, l) for l in range(5)]
    Ls = [M.MoELayer.create(M.upload(l, dev), cfg.d, cfg.f, cfg.E, cfg.k, 1, 1) for l in lays]
    X0 = tokens(cfg, OM.Layer.from_dict(lays[0]), 3, 1)
    base = torch.from_numpy(F.bf16_to_f64(X0).astype(np.float32)).to(dev)
    handles = [L.handle for L in Ls]
    stream = torch.cuda.Stream()
    re_, ie_ = torch.empty_like(base), torch.empty((5, 1, cfg.k), dtype=torch.int32, device=dev)
    rg, ig = torch.empty_like(base), torch.empty_like(ie_)

    def run(r, it):
        def step(i):
            r.copy_(base)
            M.moe_decode_stack_forward(handles, r, 1, 1e-6, None, None, it, stream)
        return step

    with torch.cuda.stream(stream):
        run(re_, ie_)(0)
    torch.cuda.synchronize()
    g = capture(run(rg, ig), 1, stream)
    replay_checked(g, [re_, ie_], [rg, ig])
    ro = OM.stack_forward([OM.Layer.from_dict(l) for l in lays], X0[0], cfg.k, 1e-6)["r"]
    err = np.abs(re_.cpu().numpy()[0].astype(np.float64) - ro).max()
    assert err <= Y_TOL * np.abs(ro).max()
    for L in Ls:
        L.close()


def test_lmhead_in_a_graph():
    """The LM head at B=8 over the full vocabulary, captured and replayed
    (its last-arrival counters reset by the kernel itself)."""
    import torch
    from oracle import lmhead as OH
    from oracle.inputs import pick_hidden_rows
    dev = device()
    cfg = synth.LMHEAD8
    q, s = synth.make_lmhead(cfg, 1)
    H, _ = pick_hidden_rows(q, s, cfg.margin, lambda b, a: synth.draw_hidden(cfg, 1, b, a), cfg.B)
    H = np.stack(H)
    wq, ws = torch.from_numpy(q).to(dev), torch.from_numpy(s.view(np.int16)).to(dev)
    x = torch.from_numpy(H.view(np.int16)).to(dev)
    wsz = M.lmhead_int4_argmax_workspace_bytes(cfg.V, cfg.d, cfg.B)
    wsp = torch.zeros(wsz, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    te, me = torch.empty(cfg.B, dtype=torch.int32, device=dev), torch.empty(cfg.B, dtype=torch.float32, device=dev)
    tg, mg = torch.empty_like(te), torch.empty_like(me)

    def run(t, m):
        def step(i):
            M.lmhead_int4_argmax(wq, ws, cfg.V, cfg.d, x, cfg.B, t, m, wsp, wsz, stream)
        return step

    with torch.cuda.stream(stream):
        run(te, me)(0)
    torch.cuda.synchronize()
    g = capture(run(tg, mg), 1, stream)
    replay_checked(g, [te, me], [tg, mg])
    tok, _, _ = OH.lmhead_argmax(q, s, H)
    assert te.cpu().numpy().tolist() == tok.tolist()
