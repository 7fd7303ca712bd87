"""The persistent stack kernel (one launch steps every workgroup through up
to 64 layers, MOE_STACK_PERSISTENT) against one launch per layer: the same
kernels' arithmetic, so every layer's x, y, chosen experts and the final
residual agree bit for bit; and against the fp64 oracle layer by layer
(teacher forcing, as in test_gpu_stack).  Also: more layers than one launch
takes, the pages' top-6 + shared layer, the FP4 formats, and the error flag
of a forced give-up in the wait for the previous layer's output."""
import numpy as np
import pytest

import synth
import sparse_moe_decode_gemv_amd as M
from gpu_common import device, tokens
from oracle import formats as F
from oracle import moe as OM
from test_gpu_stack import EPS, check_teacher_forced

pytestmark = pytest.mark.gpu


def _layers(cfg, seed, n):
    dev = device()
    lays = [synth.make_layer(cfg, seed, l) for l in range(n)]
    Ls = [M.MoELayer.create(M.upload(l, dev), cfg.d, cfg.f, cfg.E, cfg.k, 1, 1) for l in lays]
    return lays, Ls


def _run(Ls, cfg, X0, flags):
    import torch
    dev = device()
    nl = len(Ls)
    r = torch.from_numpy(F.bf16_to_f64(X0).astype(np.float32)).to(dev)
    xt = torch.zeros((nl, 1, cfg.d), dtype=torch.int16, device=dev)
    yt = torch.full((nl, 1, cfg.d), float("nan"), dtype=torch.float32, device=dev)
    it = torch.full((nl, 1, cfg.k), -1, dtype=torch.int32, device=dev)
    M.moe_decode_stack_forward_ex([L.handle for L in Ls], r, 1, EPS, xt, yt, it, flags)
    torch.cuda.synchronize()
    return r.cpu().numpy(), xt.cpu().numpy().view(np.uint16), yt.cpu().numpy(), it.cpu().numpy()


def _same(a, b):
    for u, v, what in zip(a, b, ("residual", "x trace", "y trace", "idx trace")):
        if u.dtype.kind == "f":
            u, v = u.view(np.uint32), v.view(np.uint32)
        assert np.array_equal(u, v), f"{what} differs between the persistent and per-layer stacks"


@pytest.mark.parametrize("cfg,n,seed", [(synth.STACK, 8, 1), (synth.TINY, 49, 2), (synth.TINY, 70, 3)],
                         ids=["flagship-8", "tiny-49", "tiny-70-two-launches"])
def test_persistent_equals_per_layer_and_oracle(cfg, n, seed):
    lays, Ls = _layers(cfg, seed, n)
    OLs = [OM.Layer.from_dict(l) for l in lays]
    X0 = tokens(cfg, OLs[0], seed, 1)
    per = _run(Ls, cfg, X0, 0)
    pers = _run(Ls, cfg, X0, M.MOE_STACK_PERSISTENT)
    _same(pers, per)
    again = _run(Ls, cfg, X0, M.MOE_STACK_PERSISTENT)  # repeat calls: same bits
    _same(again, pers)
    check_teacher_forced(OLs, cfg, X0, *pers)
    for L in Ls:
        assert L.error_flags() == 0
        L.close()


@pytest.mark.parametrize("cfg", [synth.FLINT, synth.LAYER_FP4, synth.LAYER_NV], ids=["top6-shared", "mxfp4", "nvfp4"])
def test_persistent_other_layers(cfg):
    """4 flagship-shape layers of the pages' routing and of both FP4 formats."""
    lays, Ls = _layers(cfg, 4, 4)
    OLs = [OM.Layer.from_dict(l) for l in lays]
    X0 = tokens(cfg, OLs[0], 4, 1)
    per = _run(Ls, cfg, X0, 0)
    pers = _run(Ls, cfg, X0, M.MOE_STACK_PERSISTENT)
    _same(pers, per)
    check_teacher_forced(OLs, cfg, X0, *pers)
    for L in Ls:
        L.close()


def test_persistent_forced_give_up_sets_flags_and_recovers():
    """Every wait of a persistent 3-layer stack looking for a tag nobody
    writes: the launch ends, layers 1 and 2 report the residual wait (bit 2)
    besides bits 0 and 1; with the default restored the next call is
    correct again."""
    cfg = synth.TINY
    lays, Ls = _layers(cfg, 5, 3)
    OLs = [OM.Layer.from_dict(l) for l in lays]
    X0 = tokens(cfg, OLs[0], 5, 1)
    M.moe_decode_set_wait_limit(Ls[0].handle, 3, 1)
    _run(Ls, cfg, X0, M.MOE_STACK_PERSISTENT)
    flags = [L.error_flags() for L in Ls]
    assert flags[0] == 3 and flags[1] == 7 and flags[2] == 7, flags
    M.moe_decode_set_wait_limit(Ls[0].handle, M.DEFAULT_WAIT_POLLS, 0)
    pers = _run(Ls, cfg, X0, M.MOE_STACK_PERSISTENT)
    per = _run(Ls, cfg, X0, 0)
    _same(pers, per)
    check_teacher_forced(OLs, cfg, X0, *pers)
    assert all(L.error_flags() == 0 for L in Ls)
    for L in Ls:
        L.close()
