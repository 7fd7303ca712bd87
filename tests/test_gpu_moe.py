"""GPU parity of the MoE layer decode step against the fp64 oracle, through
the C ABI.  Seeded synthetic inputs (synth), margin-conditioned with the
oracle so the chosen experts are unique."""
import numpy as np
import pytest

import synth
import sparse_moe_decode_gemv_amd as M
from gpu_common import Y_TOL, as_i16, compare_layer, device, tokens, zero_expert_layer
from oracle import moe as OM

pytestmark = pytest.mark.gpu


def run_layer(layer_np, cfg, X, norm=1, max_tokens=None):
    import torch
    dev = device()
    T = X.shape[0]
    L = M.MoELayer.create(M.upload(layer_np, dev), cfg.d, cfg.f, cfg.E, cfg.k, norm, max_tokens or T)
    x = torch.from_numpy(as_i16(X)).to(dev)
    y = torch.full((T, cfg.d), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.full((T, cfg.k), -1, dtype=torch.int32, device=dev)
    w = torch.full((T, cfg.k), float("nan"), dtype=torch.float32, device=dev)
    L.forward(x, y, idx, w)
    torch.cuda.synchronize()
    return L, y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5])
def test_tiny_layer_parity(seed):
    cfg = synth.TINY
    lay = synth.make_layer(cfg, seed)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, seed, 4)
    _, y, idx, w = run_layer(lay, cfg, X, max_tokens=8)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, f"tiny seed {seed}")


def test_tiny_layer_without_renormalization():
    cfg = synth.TINY
    lay = synth.make_layer(cfg, 2)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 2, 3)
    _, y, idx, w = run_layer(lay, cfg, X, norm=0)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k, norm_topk=False), idx, w, y, "tiny norm=0")


@pytest.mark.parametrize("k", [1, 3, 16])
def test_tiny_layer_other_k(k):
    from dataclasses import replace
    cfg = replace(synth.TINY, k=k)
    lay = synth.make_layer(cfg, 7)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 7, 2)
    _, y, idx, w = run_layer(lay, cfg, X)
    compare_layer(OM.moe_forward_tokens(OL, X, k), idx, w, y, f"tiny k={k}")


def test_odd_expert_count_and_bias():
    """E = 100 (not a multiple of the wave width), router bias present."""
    from dataclasses import replace
    cfg = replace(synth.TINY, E=100, k=5)
    lay = synth.make_layer(cfg, 8)
    lay["router_b"] = (np.arange(100) % 7 - 3).astype(np.float32) * 0.05
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 8, 3)
    _, y, idx, w = run_layer(lay, cfg, X)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, "E=100")


@pytest.mark.parametrize("seed", [1, 2])
def test_flagship_layer_parity(seed):
    """d=2048, f=512, E=256, top-8: every output of 3 tokens against the oracle."""
    cfg = synth.LAYER
    lay = synth.make_layer(cfg, seed)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, seed, 3)
    out = OM.moe_forward_tokens(OL, X, cfg.k)
    # one call per token, as decode runs it
    for t in range(3):
        _, y, idx, w = run_layer(lay, cfg, X[t:t + 1])
        compare_layer({k: v[t:t + 1] for k, v in out.items()}, idx, w, y, f"layer seed {seed} token {t}")


def test_batch_with_zipf_bias_parity():
    """T=64 tokens of the flagship layer with the Zipf(1.1) router bias."""
    cfg = synth.BATCH
    lay = synth.make_layer(cfg, 1)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 1, cfg.T)
    _, y, idx, w = run_layer(lay, cfg, X)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, "batch")
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    assert counts.max() >= 16  # the skew the workload is built to have


def test_ragged_token_counts_reuse_one_handle():
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
