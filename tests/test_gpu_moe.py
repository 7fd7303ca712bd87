"""GPU parity of the MoE layer decode step against the fp64 oracle, through
the C ABI.  Seeded synthetic inputs (synth), margin-conditioned with the
oracle so the chosen experts are unique."""
import numpy as np
import pytest

import synth
import sparse_moe_decode_gemv_amd as M
from gpu_common import Y_TOL, as_i16, compare_layer, device, tokens, zero_expert_layer
from oracle import cpp_oracle as OC
from oracle import moe as OM

pytestmark = pytest.mark.gpu


def run_layer(layer_np, cfg, X, norm=1, max_tokens=None, one_by_one=False):
    """All T tokens in one call (batched path), or one call per token
    (the single-launch 1-token path)."""
    import torch
    dev = device()
    T = X.shape[0]
    L = M.MoELayer.create(M.upload(layer_np, dev), cfg.d, cfg.f, cfg.E, cfg.k, norm, max_tokens or T)
    x = torch.from_numpy(as_i16(X)).to(dev)
    y = torch.full((T, cfg.d), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.full((T, cfg.k), -1, dtype=torch.int32, device=dev)
    w = torch.full((T, cfg.k), float("nan"), dtype=torch.float32, device=dev)
    if one_by_one:
        for t in range(T):
            L.forward(x[t:t + 1], y[t:t + 1], idx[t:t + 1], w[t:t + 1])
    else:
        L.forward(x, y, idx, w)
    torch.cuda.synchronize()
    return L, y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


BOTH = pytest.mark.parametrize("one_by_one", [False, True], ids=["batched", "single-launch"])


def check_groups(L, T, idx_gpu):
    """The batched path's grouping of assignments by expert, bit-exact
    against the definition applied to the chosen experts the GPU returned."""
    import torch
    dev = device()
    off = torch.full((L.E + 1,), -1, dtype=torch.int32, device=dev)
    asg = torch.full((T * L.k,), -1, dtype=torch.int32, device=dev)
    act = torch.full((L.E,), -1, dtype=torch.int32, device=dev)
    na = torch.full((1,), -1, dtype=torch.int32, device=dev)
    M.moe_decode_expert_groups(L.handle, T, off, asg, act, na)
    torch.cuda.synchronize()
    e_off, e_asg, e_act = OM.group_by_expert(idx_gpu[:T], L.E)
    assert np.array_equal(off.cpu().numpy(), e_off), "offsets"
    assert np.array_equal(asg.cpu().numpy(), e_asg), "assignment order"
    n = int(na.item())
    assert n == len(e_act) and np.array_equal(act.cpu().numpy()[:n], e_act), "active experts"


@BOTH
@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5])
def test_tiny_layer_parity(seed, one_by_one):
    cfg = synth.TINY
    lay = synth.make_layer(cfg, seed)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, seed, 4)
    L, y, idx, w = run_layer(lay, cfg, X, max_tokens=8, one_by_one=one_by_one)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, f"tiny seed {seed}")
    if not one_by_one:
        check_groups(L, 4, idx)


@BOTH
def test_tiny_layer_without_renormalization(one_by_one):
    cfg = synth.TINY
    lay = synth.make_layer(cfg, 2)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 2, 3)
    _, y, idx, w = run_layer(lay, cfg, X, norm=0, one_by_one=one_by_one)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k, norm_topk=False), idx, w, y, "tiny norm=0")


@BOTH
@pytest.mark.parametrize("k", [1, 3, 16])
def test_tiny_layer_other_k(k, one_by_one):
    from dataclasses import replace
    cfg = replace(synth.TINY, k=k)
    lay = synth.make_layer(cfg, 7)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 7, 2)
    L, y, idx, w = run_layer(lay, cfg, X, one_by_one=one_by_one)
    compare_layer(OM.moe_forward_tokens(OL, X, k), idx, w, y, f"tiny k={k}")
    if not one_by_one:
        check_groups(L, 2, idx)


@BOTH
def test_odd_expert_count_and_bias(one_by_one):
    """E = 100 (not a multiple of the wave width), router bias present."""
    from dataclasses import replace
    cfg = replace(synth.TINY, E=100, k=5)
    lay = synth.make_layer(cfg, 8)
    lay["router_b"] = (np.arange(100) % 7 - 3).astype(np.float32) * 0.05
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 8, 3)
    L, y, idx, w = run_layer(lay, cfg, X, one_by_one=one_by_one)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, "E=100")
    if not one_by_one:
        check_groups(L, 3, idx)


def test_flagship_tied_router_logits_pick_lower_expert():
    """Router rows 3 and 200 made identical and dominant: their logits tie
    exactly, and the lower expert index must come first."""
    cfg = synth.LAYER
    lay = synth.make_layer(cfg, 4)
    lay["router_w"] = lay["router_w"].copy()
    lay["router_w"][3] = lay["router_w"][200] = np.float32(0.05)
    OL = OM.Layer.from_dict(lay)
    X = np.full((1, cfg.d), 0x3F80, np.uint16)  # x = 1: both rows give the same fp32 sum
    out = OM.moe_forward_tokens(OL, X, cfg.k)
    assert OM.topk_margin(out["logits"][0], cfg.k) > 1e-3  # the rest of the set is unambiguous
    _, y, idx, w = run_layer(lay, cfg, X, one_by_one=True)
    assert idx[0][0] == 3 and idx[0][1] == 200, idx[0]
    assert w[0][0] == w[0][1]
    assert out["idx"][0][0] == 3 and out["idx"][0][1] == 200
    err = np.abs(y[0] - out["y"][0]).max()
    assert err <= 2e-3 * np.abs(out["y"][0]).max()


@pytest.mark.parametrize("one_by_one", [True, False], ids=["single-launch", "batched"])
def test_flagship_near_tied_router_logits_keep_their_order(one_by_one):
    """Rows 3 and 200 dominant and equal but for one element of row 200,
    larger by 1e-4: the two logits agree in their leading bits (the part the
    selection keys keep) and row 200 must come first, by value."""
    cfg = synth.LAYER
    lay = synth.make_layer(cfg, 4)
    lay["router_w"] = lay["router_w"].copy()
    lay["router_w"][3] = lay["router_w"][200] = np.float32(0.05)
    lay["router_w"][200, 0] = np.float32(0.05 + 1e-4)
    OL = OM.Layer.from_dict(lay)
    X = np.full((2, cfg.d), 0x3F80, np.uint16)
    out = OM.moe_forward_tokens(OL, X, cfg.k)
    assert OM.topk_margin(out["logits"][0], cfg.k) > 1e-3
    assert out["idx"][0][0] == 200 and out["idx"][0][1] == 3
    _, y, idx, w = run_layer(lay, cfg, X, one_by_one=one_by_one)
    for t in range(2):
        assert idx[t][0] == 200 and idx[t][1] == 3, idx[t]
        assert w[t][0] > w[t][1]
        compare_layer({k: v[t:t + 1] for k, v in out.items()}, idx[t:t + 1], w[t:t + 1], y[t:t + 1], f"token {t}")


@pytest.mark.parametrize("seed", [1, 2])
def test_flagship_layer_parity(seed):
    """d=2048, f=512, E=256, top-8: every output of 3 tokens against the oracle."""
    cfg = synth.LAYER
    lay = synth.make_layer(cfg, seed)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, seed, 3)
    out = OM.moe_forward_tokens(OL, X, cfg.k)
    cout = OC.moe_forward_tokens(lay, X, cfg.k)  # the plain C++ oracle
    # one call per token, as decode runs it
    for t in range(3):
        _, y, idx, w = run_layer(lay, cfg, X[t:t + 1])
        compare_layer({k: v[t:t + 1] for k, v in out.items()}, idx, w, y, f"layer seed {seed} token {t}")
        compare_layer({k: v[t:t + 1] for k, v in cout.items()}, idx, w, y, f"layer seed {seed} token {t} (C++)")


def test_batch_with_zipf_bias_parity():
    """T=64 tokens of the flagship layer with the Zipf(1.1) router bias."""
    cfg = synth.BATCH
    lay = synth.make_layer(cfg, 1)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 1, cfg.T)
    L, y, idx, w = run_layer(lay, cfg, X)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, "batch")
    compare_layer(OC.moe_forward_tokens(lay, X, cfg.k), idx, w, y, "batch (C++ oracle)")
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    assert counts.max() > 32  # the skew the workload is built to have: several 32-token chunks
    check_groups(L, cfg.T, idx)


def test_batch_repeat_calls_are_bit_identical():
    """The batched path has no atomics in its arithmetic: same input, same bits."""
    import torch
    cfg = synth.BATCH
    lay = synth.make_layer(cfg, 2)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 2, cfg.T)
    dev = device()
    L = M.MoELayer.create(M.upload(lay, dev), cfg.d, cfg.f, cfg.E, cfg.k, 1, cfg.T)
    x = torch.from_numpy(as_i16(X)).to(dev)
    outs = []
    for _ in range(5):
        y = torch.empty((cfg.T, cfg.d), device=dev)
        L.forward(x, y)
        outs.append(y.cpu().numpy())
    for y in outs[1:]:
        assert np.array_equal(y, outs[0])


@pytest.mark.parametrize("T,k", [(256, 4), (64, 16)])
def test_max_tokens_and_hot_experts(T, k):
    """Up to the largest T: with 16 experts every expert takes many 32-token
    chunks (k=16: all 16 experts chosen by every token)."""
    from dataclasses import replace
    cfg = replace(synth.TINY, k=k)
    lay = synth.make_layer(cfg, 9)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 9, T)
    L, y, idx, w = run_layer(lay, cfg, X)
    compare_layer(OM.moe_forward_tokens(OL, X, k), idx, w, y, f"T={T} k={k}")
    check_groups(L, T, idx)


@pytest.mark.parametrize("d,f,E,k,T", [(512, 256, 8, 2, 5), (1024, 1024, 4, 2, 3), (4096, 1024, 4, 2, 3),
                                       (256, 4096, 3, 1, 4), (8192, 128, 2, 1, 2)])
def test_other_shapes_batched(d, f, E, k, T):
    """Every template of the grouped kernels: K split 1, 2 or 4 ways, one or
    several passes over K."""
    from dataclasses import replace
    cfg = replace(synth.LAYER, d=d, f=f, E=E, k=k)
    lay = synth.make_layer(cfg, 11)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 11, T)
    L, y, idx, w = run_layer(lay, cfg, X)
    compare_layer(OM.moe_forward_tokens(OL, X, k), idx, w, y, f"d={d} f={f}")
    check_groups(L, T, idx)


def test_single_launch_and_batched_calls_interleave_on_one_handle():
    """T=1 calls (single launch, epoch-tagged hand-offs) and T>1 calls
    (batched kernels) alternate on the same workspace."""
    import torch
    cfg = synth.LAYER
    lay = synth.make_layer(cfg, 5)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 5, 4)
    ref = OM.moe_forward_tokens(OL, X, cfg.k)
    dev = device()
    L = M.MoELayer.create(M.upload(lay, dev), cfg.d, cfg.f, cfg.E, cfg.k, 1, 4)
    x = torch.from_numpy(as_i16(X)).to(dev)
    for rnd in range(3):
        for T in (1, 4, 1, 1, 2):
            y = torch.full((T, cfg.d), float("nan"), device=dev)
            idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
            w = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
            L.forward(x[:T], y, idx, w)
            torch.cuda.synchronize()
            compare_layer({k: v[:T] for k, v in ref.items()}, idx.cpu().numpy(), w.cpu().numpy(),
                          y.cpu().numpy(), f"round {rnd} T={T}")


def test_ragged_token_counts_reuse_one_handle():
    """T = 7, 1, 3 on one handle sized for 7; T = 8 and T = 0 are rejected."""
    import torch
    cfg = synth.TINY
    lay = synth.make_layer(cfg, 3)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 3, 7)
    dev = device()
    L = M.MoELayer.create(M.upload(lay, dev), cfg.d, cfg.f, cfg.E, cfg.k, 1, 7)
    for T in (7, 1, 3):
        x = torch.from_numpy(as_i16(X[:T])).to(dev)
        y = torch.full((T, cfg.d), float("nan"), device=dev)
        idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
        w = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
        L.forward(x, y, idx, w)
        torch.cuda.synchronize()
        compare_layer(OM.moe_forward_tokens(OL, X[:T], cfg.k), idx.cpu().numpy(), w.cpu().numpy(),
                      y.cpu().numpy(), f"T={T}")
    with pytest.raises(M.MoEError) as ei:
        L.forward(torch.zeros((8, cfg.d), dtype=torch.int16, device=dev))
    assert ei.value.status == M.MOE_ERR_SHAPE
    # an empty call (T = 0) is a shape error too, and launches nothing
    y0 = torch.full((1, cfg.d), 7.0, device=dev)
    with pytest.raises(M.MoEError) as ei:
        M.moe_decode_forward(L.handle, torch.zeros((1, cfg.d), dtype=torch.int16, device=dev), 0, y0)
    assert ei.value.status == M.MOE_ERR_SHAPE
    torch.cuda.synchronize()
    assert torch.all(y0 == 7.0)


def test_zero_scale_experts_give_zero_output_and_every_element_is_written():
    cfg = synth.TINY
    lay = zero_expert_layer(synth.make_layer(cfg, 4))
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 4, 2)
    _, y, idx, w = run_layer(lay, cfg, X)
    assert np.all(y == 0.0)  # NaN-prefilled buffer fully overwritten


def test_repeat_calls_are_bit_identical():
    import torch
    cfg = synth.LAYER
    lay = synth.make_layer(cfg, 3)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 3, 1)
    dev = device()
    L = M.MoELayer.create(M.upload(lay, dev), cfg.d, cfg.f, cfg.E, cfg.k)
    x = torch.from_numpy(as_i16(X)).to(dev)
    ys = []
    for _ in range(20):
        y = torch.empty((1, cfg.d), device=dev)
        idx = torch.empty((1, cfg.k), dtype=torch.int32, device=dev)
        L.forward(x, y, idx)
        ys.append((y.cpu().numpy(), idx.cpu().numpy()))
    for y, idx in ys[1:]:
        assert np.array_equal(y, ys[0][0]) and np.array_equal(idx, ys[0][1])
