"""Shared pieces of the GPU parity tests: seeded inputs picked with the
oracle's margin rule, device upload, and the comparison rules (chosen
experts and argmax bit-exact, y within 2e-3 * max|y|, weights within 1e-5)."""
import numpy as np

import synth
from oracle import formats as F
from oracle import moe as OM
from oracle.inputs import pick_token

Y_TOL = 2e-3      # max |y_gpu - y_oracle| <= Y_TOL * max |y_oracle|, per token
W_TOL = 1e-5      # |w_gpu - w_oracle|


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def tokens(cfg, layer, seed, T, lidx=0):
    """T margin-conditioned bf16 rows for (cfg, seed, layer index lidx)."""
    xs = [pick_token(layer, cfg.k, cfg.margin, lambda a, t=t: synth.draw_x(cfg, seed, lidx, t, a))[0]
          for t in range(T)]
    return np.stack(xs)


def as_i16(a):
    return np.ascontiguousarray(a).view(np.int16)


def compare_layer(out, idx_gpu, w_gpu, y_gpu, what=""):
    """Oracle result `out` (moe_forward_tokens) against the GPU's arrays."""
    T = y_gpu.shape[0]
    for t in range(T):
        o_idx, o_w = out["idx"][t], out["w"][t]
        order = np.argsort(o_idx)
        g_order = np.argsort(idx_gpu[t])
        assert np.array_equal(np.sort(idx_gpu[t]), o_idx[order]), f"{what} token {t}: experts {idx_gpu[t]} vs {o_idx}"
        np.testing.assert_allclose(w_gpu[t][g_order], o_w[order], rtol=0, atol=W_TOL, err_msg=f"{what} token {t} w")
        yo = out["y"][t]
        err = np.abs(y_gpu[t].astype(np.float64) - yo).max()
        assert err <= Y_TOL * np.abs(yo).max(), f"{what} token {t}: max err {err:.3e} vs {Y_TOL * np.abs(yo).max():.3e}"
        # the order of the chosen set: non-increasing weights
        assert np.all(np.diff(w_gpu[t]) <= 1e-7), f"{what} token {t}: weights not in descending order"


def zero_expert_layer(layer):
    L = dict(layer)
    L["down_s"] = np.zeros_like(layer["down_s"])
    return L
