"""GPU parity of the pre-norm stack of MoE layers (moe_decode_stack_forward)
against the fp64 oracle, checked layer by layer with teacher forcing: the
oracle re-runs layer l from the GPU's own x_l.

Only x_0 is margin-conditioned; deeper layers cannot be.  Where the
oracle's gap between the k-th and (k+1)-th logit at a layer is at least the
margin, the chosen experts must match exactly; below it the GPU's set is
accepted if each of its logits is within 1e-4 of the oracle's k-th, and
y_l is then checked against the oracle evaluated on the GPU's set."""
import numpy as np
import pytest

import synth
import sparse_moe_decode_gemv_amd as M
from gpu_common import Y_TOL, as_i16, device, tokens
from oracle import cpp_oracle as OC
from oracle import formats as F
from oracle import moe as OM

pytestmark = pytest.mark.gpu

EPS = 1e-6
CLOSE = 1e-4     # logit slack accepted for a chosen expert below the margin


def run_stack(layers_np, cfg, X0):
    import torch
    dev = device()
    T, nl = X0.shape[0], len(layers_np)
    Ls = [M.MoELayer.create(M.upload(l, dev), cfg.d, cfg.f, cfg.E, cfg.k, 1, T) for l in layers_np]
    r = torch.from_numpy(F.bf16_to_f64(X0).astype(np.float32)).to(dev)
    xt = torch.zeros((nl, T, cfg.d), dtype=torch.int16, device=dev)
    yt = torch.full((nl, T, cfg.d), float("nan"), dtype=torch.float32, device=dev)
    it = torch.full((nl, T, cfg.k), -1, dtype=torch.int32, device=dev)
    M.moe_decode_stack_forward([L.handle for L in Ls], r, T, EPS, xt, yt, it)
    torch.cuda.synchronize()
    out = r.cpu().numpy(), xt.cpu().numpy().view(np.uint16), yt.cpu().numpy(), it.cpu().numpy()
    for L in Ls:
        L.close()
    return out


def check_teacher_forced(layers_o, cfg, X0, r_gpu, xt, yt, it):
    """Returns the number of (layer, token) pairs below the margin."""
    T, d, k = X0.shape[0], cfg.d, cfg.k
    r = F.bf16_to_f64(X0).astype(np.float32)
    below = 0
    for l, OL in enumerate(layers_o):
        for t in range(T):
            where = f"layer {l} token {t}"
            # the pre-norm: the GPU normalizes in fp32, the oracle in fp64;
            # each bf16 code may differ by one unit in the last place
            xo = OM.rmsnorm_bf16(r[t], EPS)
            dx = np.abs(xo.astype(np.int32) - xt[l, t].astype(np.int32))
            assert dx.max() <= 1, f"{where}: x_l differs by {dx.max()} bf16 units"
            assert np.count_nonzero(dx) <= max(2, d // 64), f"{where}: {np.count_nonzero(dx)} x_l codes differ"
            ref = OM.moe_forward(OL, xt[l, t], k)
            gset = np.sort(it[l, t])
            assert np.all((gset >= 0) & (gset < cfg.E)) and len(np.unique(gset)) == k, f"{where}: set {it[l, t]}"
            if OM.topk_margin(ref["logits"], k) >= cfg.margin:
                assert np.array_equal(gset, np.sort(ref["idx"])), f"{where}: experts {gset} vs {np.sort(ref['idx'])}"
            else:
                below += 1
                kth = np.sort(ref["logits"])[::-1][k - 1]
                assert np.all(ref["logits"][gset] >= kth - CLOSE), f"{where}: {gset} not among the top {k}"
                ref = OM.moe_forward_on_set(OL, xt[l, t], gset)
            err = np.abs(yt[l, t].astype(np.float64) - ref["y"]).max()
            assert err <= Y_TOL * np.abs(ref["y"]).max(), f"{where}: y err {err:.3e}"
        # residual add in fp32, element by element: reproduced exactly
        r = (r + yt[l]).astype(np.float32)
    assert np.array_equal(r, r_gpu), "final residual is not r_0 + sum of the layer outputs in fp32"
    return below


def end_to_end(layers_o, cfg, X0, r_gpu):
    """Whole-stack oracles (numpy and C++) from x_0 alone: final residual
    within Y_TOL of max |r| per token (valid when no layer fell below the
    margin)."""
    layers_c = [OC.CLayer(l) for l in layers_o]
    for t in range(X0.shape[0]):
        for name, ro in (("numpy", OM.stack_forward(layers_o, X0[t], cfg.k, EPS)["r"]),
                         ("C++", OC.stack_forward(layers_c, X0[t], cfg.k, EPS)["r"])):
            ro = ro.astype(np.float64)
            err = np.abs(r_gpu[t].astype(np.float64) - ro).max()
            assert err <= Y_TOL * np.abs(ro).max(), f"token {t}: final residual err {err:.3e} ({name} oracle)"


@pytest.mark.parametrize("seed,T", [(1, 3), (2, 1), (3, 1)], ids=["T3-batched", "T1-fused-a", "T1-fused-b"])
def test_tiny_stack_49_layers(seed, T):
    """49 layers (odd: the single-launch stack ends with one residual copy)."""
    cfg = synth.TINY
    layers_np = [synth.make_layer(cfg, seed, l) for l in range(49)]
    layers_o = [OM.Layer.from_dict(l) for l in layers_np]
    X0 = tokens(cfg, layers_o[0], seed, T)
    r, xt, yt, it = run_stack(layers_np, cfg, X0)
    below = check_teacher_forced(layers_o, cfg, X0, r, xt, yt, it)
    if below == 0:
        end_to_end(layers_o, cfg, X0, r)


@pytest.mark.parametrize("L,T", [(8, 2), (8, 1), (7, 1)], ids=["L8-T2-batched", "L8-T1-fused", "L7-T1-fused"])
def test_flagship_stack_first_layers(L, T):
    """The first layers of the 49-layer stack at the flagship shape."""
    cfg = synth.STACK
    layers_np = [synth.make_layer(cfg, 1, l) for l in range(L)]
    layers_o = [OM.Layer.from_dict(l) for l in layers_np]
    X0 = tokens(cfg, layers_o[0], 1, T)
    r, xt, yt, it = run_stack(layers_np, cfg, X0)
    below = check_teacher_forced(layers_o, cfg, X0, r, xt, yt, it)
    if below == 0:
        end_to_end(layers_o, cfg, X0, r)


def test_fused_and_batched_stacks_agree():
    """The same 6 flagship layers and token through the single-launch stack
    (T=1) and the batched one (the token twice, T=2): same experts, outputs
    within the tolerance of each other."""
    import torch
    cfg = synth.STACK
    layers_np = [synth.make_layer(cfg, 2, l) for l in range(6)]
    X0 = tokens(cfg, OM.Layer.from_dict(layers_np[0]), 2, 1)
    r1, x1, y1, i1 = run_stack(layers_np, cfg, X0)
    r2, x2, y2, i2 = run_stack(layers_np, cfg, np.concatenate([X0, X0]))
    for l in range(6):
        assert np.array_equal(np.sort(i1[l, 0]), np.sort(i2[l, 0])), f"layer {l}"
        assert np.array_equal(np.sort(i2[l, 0]), np.sort(i2[l, 1]))
    assert np.abs(r1[0] - r2[0]).max() <= Y_TOL * np.abs(r2[0]).max()
    assert np.array_equal(r2[0], r2[1])


def test_stack_of_zero_layers_keeps_the_residual():
    """Layers whose down scales are all zero add exact zeros: r_L == r_0."""
    cfg = synth.TINY
    layers_np = []
    for l in range(3):
        lay = synth.make_layer(cfg, 3, l)
        lay["down_s"] = np.zeros_like(lay["down_s"])
        layers_np.append(lay)
    X0 = tokens(cfg, OM.Layer.from_dict(layers_np[0]), 3, 2)
    r, _, yt, _ = run_stack(layers_np, cfg, X0)
    assert np.array_equal(r, F.bf16_to_f64(X0).astype(np.float32))
    assert np.all(yt == 0)


def test_flagship_stack_all_49_layers_graph_and_persistent():
    """The whole 49-layer stack at the flagship shape, launched as the bench
    times it: one launch per layer captured in a HIP graph (three replays,
    with eager work between them, each bit-identical to the eager call) and
    the persistent launch (bit-identical too); every layer of the eager call
    checked against the oracle from the GPU's own x_l, and no bounded wait
    of any layer gave up."""
    import torch
    cfg = synth.STACK
    L = cfg.layers
    layers_np = [synth.make_layer(cfg, 1, l) for l in range(L)]
    layers_o = [OM.Layer.from_dict(l) for l in layers_np]
    X0 = tokens(cfg, layers_o[0], 1, 1)
    dev = device()
    Ls = [M.MoELayer.create(M.upload(l, dev), cfg.d, cfg.f, cfg.E, cfg.k, 1, 1) for l in layers_np]
    hs = [h.handle for h in Ls]
    base = torch.from_numpy(F.bf16_to_f64(X0).astype(np.float32)).to(dev)
    xt = torch.zeros((L, 1, cfg.d), dtype=torch.int16, device=dev)
    yt = torch.full((L, 1, cfg.d), float("nan"), dtype=torch.float32, device=dev)
    it = torch.full((L, 1, cfg.k), -1, dtype=torch.int32, device=dev)
    s = torch.cuda.Stream()
    r = base.clone()
    M.moe_decode_stack_forward(hs, r, 1, EPS, xt, yt, it, s)
    s.synchronize()
    r_eager = r.cpu().numpy()
    check_teacher_forced(layers_o, cfg, X0, r_eager, xt.cpu().numpy().view(np.uint16), yt.cpu().numpy(),
                         it.cpu().numpy())
    rg = torch.empty_like(base)
    with torch.cuda.stream(s):
        rg.copy_(base)
        M.moe_decode_stack_forward(hs, rg, 1, EPS, None, None, None, s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rg.copy_(base)
        M.moe_decode_stack_forward(hs, rg, 1, EPS, None, None, None, s)
    for rep in range(3):
        rg.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(rg.cpu().numpy(), r_eager), f"graph replay {rep}"
    rp = base.clone()
    M.moe_decode_stack_forward_ex(hs, rp, 1, EPS, None, None, None, M.MOE_STACK_PERSISTENT, s)
    s.synchronize()
    assert np.array_equal(rp.cpu().numpy(), r_eager), "persistent launch"
    for l, h in enumerate(Ls):
        assert h.error_flags() == 0, f"layer {l}"
    del g
    for h in Ls:
        h.close()
