"""GPU parity of the batched path at prompt-processing sizes (hundreds to
thousands of tokens per call) against the fp64 oracle."""
import numpy as np
import pytest

import synth
from gpu_common import W_TOL, compare_layer, tokens
from oracle import formats as F
from oracle import moe as OM
from test_gpu_moe import check_groups, run_layer

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
def test_prefill_512_tokens_every_output():
    """T = 512 through the flagship layer: every token's experts, weights
    and output against the oracle, and the grouping by expert bit-exact."""
    cfg = synth.LAYER
    lay = synth.make_layer(cfg, 7)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 7, 512)
    L, y, idx, w = run_layer(lay, cfg, X)
    compare_layer(OM.moe_forward_tokens(OL, X, cfg.k), idx, w, y, "prefill 512")
    check_groups(L, 512, idx)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfgname,T", [("LAYER", 2048), ("FLINT", 1024), ("LAYER", 4096)],
                         ids=["top8-2048", "top6-shared-1024", "top8-4096-max"])
def test_prefill_large_sampled(cfgname, T):
    """T up to 4096 (MOE_MAX_TOKENS) in one call: the chosen experts of every token and the
    grouping are checked in full (bit-exact sets), the outputs of 96 tokens
    spread over the call against the oracle (it evaluates each token on its
    own, so a sample bounds its time)."""
    cfg = getattr(synth, cfgname)
    lay = synth.make_layer(cfg, 8)
    OL = OM.Layer.from_dict(lay)
    X = tokens(cfg, OL, 8, T)
    L, y, idx, w = run_layer(lay, cfg, X)
    # every token's chosen set against the oracle's router + top-k (cheap)
    for t in range(T):
        l = OM.router_logits(OL, F.bf16_to_f64(X[t]))
        S, wo = OM.route(l, cfg.k)
        assert np.array_equal(np.sort(idx[t]), np.sort(S)), f"token {t}: {idx[t]} vs {S}"
        np.testing.assert_allclose(np.sort(w[t]), np.sort(wo), rtol=0, atol=W_TOL)
    check_groups(L, T, idx)
    sample = np.linspace(0, T - 1, 96).astype(int)
    out = OM.moe_forward_tokens(OL, X[sample], cfg.k)
    compare_layer(out, idx[sample], w[sample], y[sample], f"prefill {T} sample")
