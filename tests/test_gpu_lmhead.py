"""GPU parity of the 4-bit LM head with fused argmax against the fp64 oracle."""
import numpy as np
import pytest

import synth
import sparse_moe_decode_gemv_amd as M
from conftest import golden_lines
from gpu_common import as_i16, device
from oracle import cpp_oracle as OC
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


@pytest.mark.parametrize("d,B", [(256, 1), (512, 4), (2048, 16)], ids=["valu", "mfma-d512", "mfma-d2048"])
def test_v16_hand_worked_tie_goes_to_lower_row(d, B):
    """The hand-worked 16-row head (zero weights past k = 1), the same x in
    every one of B rows: the 1-2 row kernel and the 16-row MFMA tiles."""
    rows = golden_lines("lmhead_v16.txt")
    V = 16
    u = np.full((V, d), 8)
    s = np.full((V, d // 32), 0x3C00, np.uint16)
    for r in rows:
        if r[0] == "token":
            continue
        v = int(r[0])
        u[v, 0], u[v, 1] = int(r[1]) + 8, int(r[2]) + 8
        s[v, 0] = F.f64_to_f16_bits(float(r[3]))
    X = np.zeros((B, d), np.uint16)
    X[:, 0], X[:, 1] = 0x3F80, 0x4000
    tok, ml = run(F.pack_codes(u), s, X)
    assert np.all(tok == 3) and np.all(ml == 21.0), (tok, ml)


@pytest.mark.parametrize("d,B", [(2048, 6), (1024, 5), (4096, 6)], ids=["mfma-d2048", "mfma-d1024", "valu-d4096"])
def test_extreme_magnitudes_of_x(d, B):
    """Rows of x scaled by 2^100 and 2^-100 (exact in bf16): the same
    tokens as the unscaled rows and maximum logits scaled by the same power
    of two, checked against the fp64 oracle on the scaled rows."""
    V = 5000
    q, s = synth.int4_matrix(V, d, synth.key(23, "lm-scale", V, d), 0.02)
    X, _ = pick_hidden_rows(q, s, 1e-2, lambda b, a: synth.bf16(d, synth.key(23, "h", d, b, a)), 2)
    up, down = X.copy(), X.copy()
    nz = (X & 0x7FFF) != 0
    up[nz] += np.uint16(100 << 7)      # exponent field + 100
    down[nz] -= np.uint16(100 << 7)    # exponent field - 100 (no draw is that small)
    assert np.all(((X[nz] & 0x7F80) >> 7) > 100) and np.all(((X[nz] & 0x7F80) >> 7) < 155)
    Xs = np.concatenate([X, up, down] * 2)[:B]
    check(q, s, Xs, f"scaled rows d={d} B={B}")
    tok, _ = run(q, s, Xs)
    assert np.array_equal(tok[2:4], tok[0:2]) and np.array_equal(tok[4:6], tok[0:2][: len(tok) - 4])


@pytest.mark.parametrize("d,B", [(2048, 4), (2048, 2), (512, 9), (4096, 2)], ids=["mfma", "mfma-b2", "mfma-d512", "valu"])
def test_equal_rows_far_apart_lowest_index_wins(d, B):
    """The winning row of each x copied to rows in other tiles and
    workgroups, one of them below it: every copy ties bit for bit and the
    lowest index is returned."""
    V = 40000
    q, s = synth.int4_matrix(V, d, synth.key(24, "lm-tie", V, d), 0.02)
    X, _ = pick_hidden_rows(q, s, 1e-2, lambda b, a: synth.bf16(d, synth.key(24, "h", d, b, a)), B)
    otok, _, _ = OH.lmhead_argmax(q, s, X)
    for i, a in enumerate(otok):
        for c in (a // 2, (a + 12345) % V, V - 1 - i):
            if c not in otok:
                q[c], s[c] = q[a], s[a]
    tok2, _, z = OH.lmhead_argmax(q, s, X)
    assert np.all(tok2 <= otok) and np.any(tok2 < otok)
    for b in range(B):   # apart from exact copies, the gap still holds
        m = z[b].max()
        assert m - z[b][z[b] < m].max() >= 1e-2
    check(q, s, X, f"copied rows d={d} B={B}")


@pytest.mark.parametrize("V,d,B", [(1000, 256, 1), (4099, 512, 3), (20000, 2048, 8), (3000, 4096, 2),
                                   (777, 2048, 16), (6007, 1024, 7), (33, 2048, 3), (50001, 1024, 12),
                                   (9001, 1024, 2), (300, 512, 2)])
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
    # and against the plain C++ oracle
    tok, ml = run(q, s, X)
    ctok, cml, _ = OC.lmhead_argmax(q, s, X, want_logits=False)
    assert np.array_equal(tok, ctok), f"lmhead B={B}: tokens {tok} vs C++ oracle {ctok}"
    assert np.all(np.abs(ml - cml) <= 2e-3 * np.abs(cml)), f"lmhead B={B}: max logit {ml} vs {cml}"
