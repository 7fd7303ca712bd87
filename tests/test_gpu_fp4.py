"""GPU parity of layers with MXFP4 expert weights (FP4 E2M1 codes, one E8M0
scale byte per 32 elements) against the fp64 oracle, on the single-launch
1-token step, the batched path (decode batches and prompt sizes) and the
pre-normed stack: chosen experts bit-exact, y within 2e-3 * max |y|; and
the exactness of the power-of-two block scales."""
import numpy as np
import pytest

import synth
from gpu_common import W_TOL, compare_layer, tokens
from oracle import formats as F
from oracle import moe as OM
from test_gpu_moe import BOTH, check_groups, run_layer
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


@BOTH
def test_tiny_fp4_batched_and_single(one_by_one):
    """The same MXFP4 layer handle (max_tokens 8) run as one batched call of
    4 tokens and as 4 single-launch steps."""
    cfg = synth.TINY_FP4
    lay = synth.make_layer(cfg, 4)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 4, 4)
    L, y, idx, w = run_layer(lay, cfg, X, max_tokens=8, one_by_one=one_by_one)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, "tiny fp4")
    if not one_by_one:
        check_groups(L, 4, idx)


def test_fp4_batch_zipf_64_tokens():
    """The batched call at T = 64 with the Zipf router bias (32-token chunks,
    MFMA tiles dequantized from E2M1 with the block scale folded in)."""
    cfg = synth.BATCH_FP4
    lay = synth.make_layer(cfg, 2)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 2, cfg.T)
    L, y, idx, w = run_layer(lay, cfg, X)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, "fp4 batch")
    check_groups(L, cfg.T, idx)


@pytest.mark.timeout(900)
def test_fp4_prefill_1024_sampled():
    """T = 1024 (64-token chunks): every token's chosen set and the grouping
    in full, the outputs of 64 tokens spread over the call."""
    cfg = synth.LAYER_FP4
    lay = synth.make_layer(cfg, 9)
    OL = OM.Layer.from_dict(lay)
    T = 1024
    X = tokens(cfg, OL, 9, T)
    L, y, idx, w = run_layer(lay, cfg, X)
    for t in range(T):
        S, wo = OM.route(OM.router_logits(OL, F.bf16_to_f64(X[t])), cfg.k)
        assert np.array_equal(np.sort(idx[t]), np.sort(S)), f"token {t}: {idx[t]} vs {S}"
        np.testing.assert_allclose(np.sort(w[t]), np.sort(wo), rtol=0, atol=W_TOL)
    check_groups(L, T, idx)
    sample = np.linspace(0, T - 1, 64).astype(int)
    compare_layer(OM.moe_forward_tokens(OL, X[sample], cfg.k), idx[sample], w[sample], y[sample], "fp4 prefill")


def test_fp4_batched_stack():
    """Two tokens through a pre-normed stack of 3 MXFP4 layers (the batched
    path with the pre-norm kernel)."""
    cfg = synth.LAYER_FP4
    layers_np = [synth.make_layer(cfg, 6, l) for l in range(3)]
    layers_o = [OM.Layer.from_dict(l) for l in layers_np]
    X0 = tokens(cfg, layers_o[0], 6, 2)
    r, xt, yt, it = run_stack(layers_np, cfg, X0)
    below = check_teacher_forced(layers_o, cfg, X0, r, xt, yt, it)
    if below == 0:
        end_to_end(layers_o, cfg, X0, r)
