"""GPU parity of layers with an always-on shared expert (the pages' own
routing: top-6 of 256 routed experts plus one shared expert) against the
fp64 oracle, on the single-launch 1-token path, the batched path and the
pre-normed stack."""
import numpy as np
import pytest

import synth
import sparse_moe_decode_gemv_amd as M
from gpu_common import compare_layer, device, tokens
from oracle import moe as OM
from test_gpu_moe import BOTH, check_groups, run_layer
from test_gpu_stack import check_teacher_forced, end_to_end, run_stack

pytestmark = pytest.mark.gpu


@BOTH
@pytest.mark.parametrize("seed", [1, 2])
def test_tiny_layer_with_shared_expert(seed, one_by_one):
    cfg = synth.TINY_SHARED
    lay = synth.make_layer(cfg, seed)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, seed, 3)
    L, y, idx, w = run_layer(lay, cfg, X, one_by_one=one_by_one)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, f"tiny shared seed {seed}")
    if not one_by_one:
        check_groups(L, 3, idx)


@BOTH
def test_flint_layer_top6_plus_shared(one_by_one):
    """d=2048, f=512, 256 routed experts, top-6 plus the shared expert."""
    cfg = synth.FLINT
    lay = synth.make_layer(cfg, 1)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 1, 3)
    L, y, idx, w = run_layer(lay, cfg, X, one_by_one=one_by_one)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, "flint layer")
    if not one_by_one:
        check_groups(L, 3, idx)


def test_flint_batch_zipf_64_tokens():
    """The batched call at T=64 with the Zipf router bias: the shared
    expert's two chunks of 32 tokens run beside the routed chunks."""
    cfg = synth.FLINT_BATCH
    lay = synth.make_layer(cfg, 2)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 2, cfg.T)
    L, y, idx, w = run_layer(lay, cfg, X)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, "flint batch")
    check_groups(L, cfg.T, idx)


@BOTH
def test_shared_expert_only_output(one_by_one):
    """Routed experts with zero down scales: y is the shared expert's output
    alone (and the routed choice is still reported)."""
    cfg = synth.FLINT
    lay = synth.make_layer(cfg, 3)
    lay["down_s"] = np.zeros_like(lay["down_s"])
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 3, 2)
    _, y, idx, w = run_layer(lay, cfg, X, one_by_one=one_by_one)
    out = OM.moe_forward_tokens(OL, X, cfg.k)
    compare_layer(out, idx, w, y, "shared only")
    assert np.abs(y).max() > 0


@pytest.mark.parametrize("L,T", [(4, 1), (4, 2)], ids=["fused", "batched"])
def test_flint_stack_first_layers(L, T):
    cfg = synth.FLINT
    layers_np = [synth.make_layer(cfg, 1, l) for l in range(L)]
    layers_o = [OM.Layer.from_dict(l) for l in layers_np]
    X0 = tokens(cfg, layers_o[0], 1, T)
    r, xt, yt, it = run_stack(layers_np, cfg, X0)
    below = check_teacher_forced(layers_o, cfg, X0, r, xt, yt, it)
    if below == 0:
        end_to_end(layers_o, cfg, X0, r)
