"""GPU parity of the 4-bit LM head with fused argmax against the fp64 oracle."""
import numpy as np
import pytest

import synth
import sparse_moe_decode_gemv_amd as M
from conftest import golden_lines
from gpu_common import as_i16, device
from oracle import formats as F
from oracle import lmhead as OH
from oracle.inputs import pick_hidden_rows

pytestmark = pytest.mark.gpu


def run(q, s, X):
    import torch
    dev = device()
    wq = torch.from_numpy(q).to(dev)
    ws = torch.from_numpy(as_i16(s)).to(dev)
    x = torch.from_numpy(as_i16(X)).to(dev)
    tok, ml = M.lmhead_argmax(wq, ws, x)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), ml.cpu().numpy()


def check(q, s, X, what):
    tok, ml = run(q, s, X)
    otok, oml, z = OH.lmhead_argmax(q, s, X)
    assert np.array_equal(tok, otok), f"{what}: tokens {tok} vs {otok}"
    tol = 2e-3 * np.abs(z).max(axis=1)
    assert np.all(np.abs(ml - oml) <= tol), f"{what}: max logit {ml} vs {oml}"


def test_v16_hand_worked_tie_goes_to_lower_row():
    rows = golden_lines("lmhead_v16.txt")
    V, d = 16, 256
    u = np.full((V, d), 8)
    s = np.full((V, d // 32), 0x3C00, np.uint16)
    for r in rows:
        if r[0] == "token":
            continue
        v = int(r[0])
        u[v, 0], u[v, 1] = int(r[1]) + 8, int(r[2]) + 8
        s[v, 0] = F.f64_to_f16_bits(float(r[3]))
    X = np.zeros((1, d), np.uint16)
    X[0, 0], X[0, 1] = 0x3F80, 0x4000
    tok, ml = run(F.pack_codes(u), s, X)
    assert tok[0] == 3 and ml[0] == 21.0


@pytest.mark.parametrize("V,d,B", [(1000, 256, 1), (4099, 512, 3), (20000, 2048, 8), (3000, 4096, 2),
                                   (777, 2048, 16)])
def test_small_heads_ragged_rows(V, d, B):
    q, s = synth.int4_matrix(V, d, synth.key(21, "lm-small", V, d), 0.02)
    X, _ = pick_hidden_rows(q, s, 1e-2, lambda b, a: synth.bf16(d, synth.key(21, "h", V, d, b, a)), B)
    check(q, s, X, f"V={V} d={d} B={B}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("B", [1, 8])
def test_full_lmhead_parity(B):
    """V=131072, d=2048 at batch 1 and 8, the configuration the bench times."""
    cfg = synth.LMHEAD8 if B == 8 else synth.LMHEAD1
    q, s = synth.make_lmhead(cfg, 1)
    X, _ = pick_hidden_rows(q, s, cfg.margin, lambda b, a: synth.draw_hidden(cfg, 1, b, a), B)
    check(q, s, X, f"lmhead B={B}")
