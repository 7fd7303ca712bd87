"""Error reporting of the single-launch layer step and the stack's choice
of path per layer.

The single-launch kernel's waits are bounded; a wait that gives up sets a
flag that moe_decode_error_flags reports.  The give-up is forced from the
host (moe_decode_set_wait_limit: a few polls, looking for a tag no
workgroup writes), so every kernel still ends normally.  A stack may mix
layers that run as one launch with layers that need the batched kernels;
each layer takes its own path and the result is checked against the fp64
oracle layer by layer."""
import numpy as np
import pytest

import synth
import sparse_moe_decode_gemv_amd as M
from dataclasses import replace
from gpu_common import Y_TOL, as_i16, device, tokens
from oracle import formats as F
from oracle import moe as OM
from test_gpu_stack import EPS, check_teacher_forced

pytestmark = pytest.mark.gpu


def _tiny_layer(dev, seed=4, max_tokens=1):
    cfg = synth.TINY
    lay = synth.make_layer(cfg, seed)
    return cfg, lay, M.MoELayer.create(M.upload(lay, dev), cfg.d, cfg.f, cfg.E, cfg.k, 1, max_tokens)


def test_flags_are_zero_after_normal_calls():
    import torch
    dev = device()
    cfg, lay, L = _tiny_layer(dev)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 4, 3)
    y = torch.empty((1, cfg.d), dtype=torch.float32, device=dev)
    for t in range(3):
        L.forward(torch.from_numpy(as_i16(X[t:t + 1])).to(dev), y)
    assert L.error_flags(clear=False) == 0
    assert L.error_flags() == 0
    L.close()


@pytest.mark.parametrize("polls", [1, 4])
def test_forced_timeouts_set_both_flags_and_the_next_call_is_correct(polls):
    """With every wait looking for a tag nobody writes, the call still ends
    and both flags are set; clearing resets them; with the default limit
    restored the next call matches the oracle and raises no flag."""
    import torch
    dev = device()
    cfg, lay, L = _tiny_layer(dev, seed=5)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 5, 2)
    xd = torch.from_numpy(as_i16(X)).to(dev)
    y = torch.empty((1, cfg.d), dtype=torch.float32, device=dev)
    idx = torch.empty((1, cfg.k), dtype=torch.int32, device=dev)
    M.moe_decode_set_wait_limit(L.handle, polls, 1)
    L.forward(xd[0:1], y, idx)
    torch.cuda.synchronize()
    assert L.error_flags(clear=False) == 3
    assert L.error_flags() == 3
    assert L.error_flags() == 0
    M.moe_decode_set_wait_limit(L.handle, M.DEFAULT_WAIT_POLLS, 0)
    L.forward(xd[1:2], y, idx)
    torch.cuda.synchronize()
    assert L.error_flags() == 0
    out = OM.moe_forward_tokens(OL, X[1:2], cfg.k)
    assert np.array_equal(np.sort(idx.cpu().numpy()[0]), np.sort(out["idx"][0]))
    err = np.abs(y.cpu().numpy()[0].astype(np.float64) - out["y"][0]).max()
    assert err <= Y_TOL * np.abs(out["y"][0]).max()
    with pytest.raises(M.MoEError):
        M.moe_decode_set_wait_limit(L.handle, 0, 0)
    L.close()


@pytest.mark.parametrize("order", ["fused-batched-fused", "batched-fused"])
def test_mixed_stack_takes_each_layers_path(order):
    """Tiny layers at T = 1: f = 128 runs as one launch (max_tokens = 1, no
    tile-major copy), f = 256 has no single-launch kernel and runs the
    batched kernels.  Two orders, ending in the caller's residual buffer and
    in the spare one (then copied back)."""
    import torch
    dev = device()
    base = synth.TINY
    wide = replace(base, f=256)
    cfgs = [base, wide, base] if order == "fused-batched-fused" else [wide, base]
    layers_np = [synth.make_layer(c, 6, l) for l, c in enumerate(cfgs)]
    layers_o = [OM.Layer.from_dict(l) for l in layers_np]
    Ls = [M.MoELayer.create(M.upload(l, dev), c.d, c.f, c.E, c.k, 1, 1) for l, c in zip(layers_np, cfgs)]
    X0 = tokens(base, layers_o[0], 6, 1)
    nl = len(Ls)
    r = torch.from_numpy(F.bf16_to_f64(X0).astype(np.float32)).to(dev)
    xt = torch.zeros((nl, 1, base.d), dtype=torch.int16, device=dev)
    yt = torch.full((nl, 1, base.d), float("nan"), dtype=torch.float32, device=dev)
    it = torch.full((nl, 1, base.k), -1, dtype=torch.int32, device=dev)
    M.moe_decode_stack_forward([L.handle for L in Ls], r, 1, EPS, xt, yt, it)
    torch.cuda.synchronize()
    check_teacher_forced(layers_o, base, X0, r.cpu().numpy(), xt.cpu().numpy().view(np.uint16), yt.cpu().numpy(),
                         it.cpu().numpy())
    for L in Ls:
        assert L.error_flags() == 0
        L.close()
