"""Pins of the LM-head oracle: a 16-row example worked by hand (with a tie),
a planted winning row, and the argmax against all logits."""
import numpy as np

import synth
from conftest import golden_lines
from oracle import formats as F
from oracle import lmhead as H


def test_v16_hand_worked_with_tie():
    rows = golden_lines("lmhead_v16.txt")
    table = [r for r in rows if r[0] != "token"]
    token = int([r for r in rows if r[0] == "token"][0][1])
    V, d = 16, 128
    u = np.full((V, d), 8)
    s = np.full((V, d // 32), 0x3C00, np.uint16)
    z_want = np.zeros(V)
    for v, a, b, sv, z in table:
        v = int(v)
        u[v, 0], u[v, 1] = int(a) + 8, int(b) + 8
        s[v, 0] = F.f64_to_f16_bits(float(sv))
        z_want[v] = float(z)
    x = np.zeros((1, d), np.uint16)
    x[0, 0], x[0, 1] = 0x3F80, 0x4000          # bf16 1.0 and 2.0
    tok, zmax, z = H.lmhead_argmax(F.pack_codes(u), s, x)
    np.testing.assert_array_equal(z[0], z_want)
    assert tok[0] == token and zmax[0] == 21.0


def test_planted_row_wins():
    """Row v* set to the sign pattern of x at full scale dominates every
    N(0, 0.02) row: its logit is ~7 * s * sum|x| against ~0.02 * |x| * 2."""
    cfg = synth.LMHeadConfig("t", V=4096, d=256, B=1)
    q, s = synth.int4_matrix(cfg.V, cfg.d, synth.key(11, "lmhead-test"), cfg.sigma)
    x = synth.bf16(cfg.d, synth.key(11, "hidden-test"))
    xf = F.bf16_to_f64(x)
    vstar = 1234
    u = F.unpack_codes(q, cfg.d)
    u[vstar] = np.where(xf >= 0, 15, 1)
    q2 = q.copy()
    q2[vstar] = F.pack_codes(u[vstar][None])[0]
    s2 = s.copy()
    s2[vstar] = F.f64_to_f16_bits(0.05)
    tok, zmax, z = H.lmhead_argmax(q2, s2, x[None])
    assert tok[0] == vstar
    assert np.isclose(zmax[0], F.f16_to_f64(s2[vstar, 0]) * 7 * np.abs(xf).sum(), rtol=1e-12)


def test_argmax_is_first_maximum_and_matches_sorted_logits():
    z = np.array([[0.1, 0.7, 0.3, 0.7], [5.0, -1.0, 5.0, 4.9]])
    tok, zmax = H.argmax_lowest(z)
    assert tok.tolist() == [1, 0] and zmax.tolist() == [0.7, 5.0]
    np.testing.assert_allclose(H.top2_gap(z), [0.0, 0.0])
    assert np.isclose(H.top2_gap(np.array([1.0, 3.0, 2.5]))[0], 0.5)


def test_chunking_does_not_change_logits():
    q, s = synth.int4_matrix(1000, 256, synth.key(12, "chunk"), 0.02)
    x = synth.bf16(256, synth.key(12, "x"))[None]
    z1 = H.lmhead_logits(q, s, x, rows_per_chunk=7)
    W = F.dequant(q, s, 256)
    z2 = np.array([[float(np.dot(W[v], F.bf16_to_f64(x[0]))) for v in range(1000)]])
    np.testing.assert_allclose(z1, z2, rtol=0, atol=1e-15)
