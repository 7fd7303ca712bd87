"""GPU parity of layers with MXFP4 expert weights (FP4 E2M1 codes, one E8M0
scale byte per 32 elements) against the fp64 oracle, on the single-launch
1-token step and the pre-normed stack: chosen experts bit-exact, y within
2e-3 * max |y|; and the exactness of the power-of-two block scales."""
import numpy as np
import pytest

import synth
from gpu_common import compare_layer, tokens
from oracle import moe as OM
from test_gpu_moe import run_layer
from test_gpu_stack import check_teacher_forced, end_to_end, run_stack

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", [1, 2])
def test_tiny_fp4_layer(seed):
    cfg = synth.TINY_FP4
    lay = synth.make_layer(cfg, seed)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, seed, 3)
    _, y, idx, w = run_layer(lay, cfg, X, max_tokens=1, one_by_one=True)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, f"tiny fp4 seed {seed}")


def test_flagship_fp4_layer():
    """d=2048, f=512, E=256, top-8 with MXFP4 experts."""
    cfg = synth.LAYER_FP4
    lay = synth.make_layer(cfg, 1)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 1, 3)
    _, y, idx, w = run_layer(lay, cfg, X, max_tokens=1, one_by_one=True)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, "layer fp4")


def test_flint_fp4_top6_plus_shared():
    """The pages' routing (top-6 + shared expert) with MXFP4 experts."""
    cfg = synth.FLINT_FP4
    lay = synth.make_layer(cfg, 2)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 2, 2)
    _, y, idx, w = run_layer(lay, cfg, X, max_tokens=1, one_by_one=True)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, "flint fp4")


def test_fp4_scales_are_exact_powers_of_two():
    """Raising every down scale byte by 3 leaves the chosen experts alone and
    multiplies y by exactly 8: the kernel applies 2^(b-127) exactly (ldexp
    on the fp32 block sums).  Down scales 2^-40 and 2^20 times the drawn
    ones still give the oracle's answer."""
    cfg = synth.LAYER_FP4
    lay = synth.make_layer(cfg, 3)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 3, 2)
    _, y, idx, _ = run_layer(lay, cfg, X, max_tokens=1, one_by_one=True)
    lay8 = dict(lay, down_s=(lay["down_s"].astype(np.int64) + 3).astype(np.uint8))
    _, y8, idx8, _ = run_layer(lay8, cfg, X, max_tokens=1, one_by_one=True)
    assert np.array_equal(idx, idx8)
    assert np.array_equal(y8, 8.0 * y)
    # scales far from 1: all blocks 2^-40 and 2^+20 relative, still the oracle's answer
    for shift in (-40, 20):
        lays = dict(lay, down_s=(lay["down_s"].astype(np.int64) + shift).astype(np.uint8))
        _, ys, idxs, ws = run_layer(lays, cfg, X, max_tokens=1, one_by_one=True)
        compare_layer(OM.moe_forward_tokens(OM.Layer.from_dict(lays), X, cfg.k), idxs, ws, ys, f"shift {shift}")


@pytest.mark.parametrize("L", [4])
def test_fp4_stack_first_layers(L):
    """A pre-normed stack of MXFP4 layers at the flagship shape, checked
    layer by layer with teacher forcing."""
    cfg = synth.LAYER_FP4
    layers_np = [synth.make_layer(cfg, 1, l) for l in range(L)]
    layers_o = [OM.Layer.from_dict(l) for l in layers_np]
    X0 = tokens(cfg, layers_o[0], 1, 1)
    r, xt, yt, it = run_stack(layers_np, cfg, X0)
    below = check_teacher_forced(layers_o, cfg, X0, r, xt, yt, it)
    if below == 0:
        end_to_end(layers_o, cfg, X0, r)
