"""GPU parity of layers with FP4 expert weights against the fp64 oracle, in
both FP4 formats: MXFP4 (E2M1 codes, one E8M0 scale byte per 32 elements)
and NVFP4 (E2M1 codes, one E4M3 scale byte per 16 elements, one fp32 scale
per expert matrix), on the single-launch 1-token step, the batched path
(decode batches and prompt sizes) and the pre-normed stack: chosen experts
bit-exact, y within 2e-3 * max |y|; and the exactness of MXFP4's
power-of-two block scales."""
import numpy as np
import pytest

import synth
from gpu_common import W_TOL, compare_layer, tokens
from oracle import formats as F
from oracle import moe as OM
from test_gpu_moe import BOTH, check_groups, run_layer
from test_gpu_stack import check_teacher_forced, end_to_end, run_stack

pytestmark = pytest.mark.gpu

# workload name of each format's configs: TINY_FP4 / TINY_NV, ...
FMTS = pytest.mark.parametrize("fmt", ["FP4", "NV"], ids=["mxfp4", "nvfp4"])


def cfg_of(base, fmt):
    return getattr(synth, f"{base}_{fmt}")


@FMTS
@pytest.mark.parametrize("seed", [1, 2])
def test_tiny_fp4_layer(seed, fmt):
    cfg = cfg_of("TINY", fmt)
    lay = synth.make_layer(cfg, seed)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, seed, 3)
    _, y, idx, w = run_layer(lay, cfg, X, max_tokens=1, one_by_one=True)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, f"tiny {fmt} seed {seed}")


@FMTS
def test_flagship_fp4_layer(fmt):
    """d=2048, f=512, E=256, top-8 with FP4 experts."""
    cfg = cfg_of("LAYER", fmt)
    lay = synth.make_layer(cfg, 1)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 1, 3)
    _, y, idx, w = run_layer(lay, cfg, X, max_tokens=1, one_by_one=True)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, f"layer {fmt}")


@FMTS
@BOTH
def test_flint_fp4_top6_plus_shared(fmt, one_by_one):
    """The pages' routing (top-6 + shared expert) with FP4 experts, as
    single-launch steps and as one batched call."""
    cfg = cfg_of("FLINT", fmt)
    lay = synth.make_layer(cfg, 2)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 2, 2)
    _, y, idx, w = run_layer(lay, cfg, X, max_tokens=2, one_by_one=one_by_one)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, f"flint {fmt}")


def test_mxfp4_scales_are_exact_powers_of_two():
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
    for shift in (-40, 20):
        lays = dict(lay, down_s=(lay["down_s"].astype(np.int64) + shift).astype(np.uint8))
        _, ys, idxs, ws = run_layer(lays, cfg, X, max_tokens=1, one_by_one=True)
        compare_layer(OM.moe_forward_tokens(OM.Layer.from_dict(lays), X, cfg.k), idxs, ws, ys, f"shift {shift}")


def test_nvfp4_matrix_scale_is_linear():
    """NVFP4: doubling every down matrix scale doubles y exactly on the
    single-launch step (the scale multiplies each piece's fp32 sum: exact
    for a power of two)."""
    cfg = synth.LAYER_NV
    lay = synth.make_layer(cfg, 3)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 3, 2)
    _, y, idx, _ = run_layer(lay, cfg, X, max_tokens=1, one_by_one=True)
    lay2 = dict(lay, down_ts=(lay["down_ts"] * 2).astype(np.float32))
    _, y2, idx2, _ = run_layer(lay2, cfg, X, max_tokens=1, one_by_one=True)
    assert np.array_equal(idx, idx2) and np.array_equal(y2, 2.0 * y)


@FMTS
def test_fp4_stack_first_layers(fmt):
    """A pre-normed stack of 4 FP4 layers at the flagship shape, checked
    layer by layer with teacher forcing."""
    cfg = cfg_of("LAYER", fmt)
    layers_np = [synth.make_layer(cfg, 1, l) for l in range(4)]
    layers_o = [OM.Layer.from_dict(l) for l in layers_np]
    X0 = tokens(cfg, layers_o[0], 1, 1)
    r, xt, yt, it = run_stack(layers_np, cfg, X0)
    below = check_teacher_forced(layers_o, cfg, X0, r, xt, yt, it)
    if below == 0:
        end_to_end(layers_o, cfg, X0, r)


@FMTS
@BOTH
def test_tiny_fp4_batched_and_single(fmt, one_by_one):
    """The same FP4 layer handle (max_tokens 8) run as one batched call of
    4 tokens and as 4 single-launch steps."""
    cfg = cfg_of("TINY", fmt)
    lay = synth.make_layer(cfg, 4)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 4, 4)
    L, y, idx, w = run_layer(lay, cfg, X, max_tokens=8, one_by_one=one_by_one)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, f"tiny {fmt}")
    if not one_by_one:
        check_groups(L, 4, idx)


@FMTS
def test_fp4_batch_zipf_64_tokens(fmt):
    """The batched call at T = 64 with the Zipf router bias (32-token chunks,
    MFMA tiles dequantized from E2M1 with the block scale folded in)."""
    cfg = cfg_of("BATCH", fmt)
    lay = synth.make_layer(cfg, 2)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 2, cfg.T)
    L, y, idx, w = run_layer(lay, cfg, X)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, f"batch {fmt}")
    check_groups(L, cfg.T, idx)


@FMTS
@pytest.mark.timeout(900)
def test_fp4_prefill_1024_sampled(fmt):
    """T = 1024 (64-token chunks): every token's chosen set and the grouping
    in full, the outputs of 48 tokens spread over the call."""
    cfg = cfg_of("LAYER", fmt)
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
    sample = np.linspace(0, T - 1, 48).astype(int)
    compare_layer(OM.moe_forward_tokens(OL, X[sample], cfg.k), idx[sample], w[sample], y[sample], f"prefill {fmt}")


@FMTS
def test_fp4_batched_stack(fmt):
    """Two tokens through a pre-normed stack of 3 FP4 layers (the batched
    path with the pre-norm kernel)."""
    cfg = cfg_of("LAYER", fmt)
    layers_np = [synth.make_layer(cfg, 6, l) for l in range(3)]
    layers_o = [OM.Layer.from_dict(l) for l in layers_np]
    X0 = tokens(cfg, layers_o[0], 6, 2)
    r, xt, yt, it = run_stack(layers_np, cfg, X0)
    below = check_teacher_forced(layers_o, cfg, X0, r, xt, yt, it)
    if below == 0:
        end_to_end(layers_o, cfg, X0, r)
