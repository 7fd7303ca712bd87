"""Pins of the plain C++ oracle (oracle/cpp/): the same kinds of pins as the
numpy oracle's -- textbook bit patterns, library decoders, the stored layout
and quantizer worked by hand, brute force over tiny inputs, the hand-worked
SwiGLU expert, stack and LM head, closed forms and invariants -- none of
which compute the expected value with the C++ code under test.  Last, the
two oracles, written independently, agree on seeded layers of every format.
"""
import math
from itertools import combinations

import numpy as np
import pytest

import synth
from conftest import golden_lines
from oracle import cpp_oracle as C
from oracle import moe as M  # only as a layer container and for the cross-check


def tiny(cfg=synth.TINY, seed=1):
    return synth.make_layer(cfg, seed)


def tiny_x(lay, cfg=synth.TINY, seed=1, token=0):
    """First draw whose top-k margin holds (margins taken on the C++ logits)."""
    for a in range(1000):
        x = synth.draw_x(cfg, seed, 0, token, a)
        routed = {k: v for k, v in lay.items() if not k.startswith("shared")}
        l = np.sort(C.router_logits(routed, x))[::-1]
        if l[cfg.k - 1] - l[cfg.k] >= cfg.margin:
            return x
    raise RuntimeError("no draw met the margin")


# ------------------------------------------------------------------ formats


def test_bf16_and_f16_textbook_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x4049, 0x0001, 0x7F7F], np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 3.140625, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127]
    np.testing.assert_array_equal(C.bf16_to_f64(bits), want)
    bits = np.array([0x3C00, 0x0001, 0x7BFF, 0x0400, 0x3555, 0xC000, 0x03FF, 0x2E66], np.uint16)
    want = [1.0, 2.0 ** -24, 65504.0, 2.0 ** -14, 0.333251953125, -2.0, 1023 * 2.0 ** -24, 0.0999755859375]
    np.testing.assert_array_equal(C.f16_to_f64(bits), want)


def test_decoders_match_numpy_on_every_pattern():
    """bf16 against numpy's binary32 view, binary16 against numpy's float16,
    for every bit pattern (finite ones for binary16, plus inf and NaN)."""
    b = np.arange(65536, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        ref32 = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(C.bf16_to_f64(b), ref32)
    np.testing.assert_array_equal(C.f16_to_f64(b), b.view(np.float16).astype(np.float64))


def test_encoders_round_to_nearest_even():
    b = np.arange(65536, dtype=np.uint16)
    b = b[(b & 0x7C00) != 0x7C00]
    np.testing.assert_array_equal(C.f64_to_f16_bits(C.f16_to_f64(b)), b)  # every finite value back
    x = np.random.default_rng(0).standard_normal(20000) * np.exp2(np.random.default_rng(1).integers(-30, 16, 20000))
    with np.errstate(over="ignore"):
        ref16 = x.astype(np.float16).view(np.uint16)  # overflow to inf, as the encoder does
    np.testing.assert_array_equal(C.f64_to_f16_bits(x), ref16)
    one_ulp = 2.0 ** -10
    assert C.f64_to_f16_bits([1.0 + one_ulp / 2, 1.0 + 3 * one_ulp / 2, 2.0 ** -25, 3 * 2.0 ** -25]).tolist() == \
        [0x3C00, 0x3C02, 0x0000, 0x0002]
    assert C.f64_to_bf16_bits([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -30,
                               -3.140625]).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC049]
    # bf16 of a binary32 value: round the low 16 bits to nearest even
    f = (np.random.default_rng(2).standard_normal(20000) * 3).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(C.f64_to_bf16_bits(f.astype(np.float64)), want)


def test_fp4_scale_decoders():
    rows = golden_lines("fp4_e2m1.txt")
    codes = np.array([int(r[0]) for r in rows], np.uint8)
    want = np.array([float(r[1]) for r in rows])
    got = C.e2m1_to_f64(codes)
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))
    b = np.arange(256)
    e8 = C.e8m0_to_f64(b.astype(np.uint8))
    w8 = np.empty(256)
    w8[1:255] = (b[1:255].astype(np.uint32) << 23).view(np.float32)
    w8[0] = np.array([0x00400000], np.uint32).view(np.float32)[0]
    assert np.array_equal(e8[:255], w8[:255]) and np.isnan(e8[255])


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = C.e4m3_to_f64(b)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("pattern", ["A", "B"])
def test_int4_layout_hand_worked(pattern):
    rows = {ln[0]: bytes(int(h, 16) for h in ln[1:]) for ln in golden_lines("int4_layout_k128.txt")}
    k = np.arange(128)
    u = (k // 8) % 16 if pattern == "A" else k % 8 + 8 * (k // 64)
    assert C.pack_codes(u[None, :])[0].tobytes() == rows[pattern]
    np.testing.assert_array_equal(C.unpack_codes(np.frombuffer(rows[pattern], np.uint8)[None], 128)[0], u)


def test_quantize_hand_worked_group_and_round_trip():
    lines = {ln[0]: ln[1:] for ln in golden_lines("quantize_group.txt")}
    w = np.array([float(v) for v in lines["w"]], np.float32)
    u, s = C.quantize(w[None, :])
    assert int(s[0, 0]) == int(lines["scale_bits"][0], 16)
    np.testing.assert_array_equal(u[0], [int(v) for v in lines["u"]])
    # quantize(dequant(q, s)) == (q, s) when every group reaches |q| = 7 and s is normal
    rng = np.random.default_rng(1)
    R, K = 64, 256
    q = rng.integers(-7, 8, size=(R, K))
    q[:, ::32] = np.where(rng.random((R, K // 32)) < 0.5, 7, -7)
    sb = rng.integers(0x0400, 0x7800, size=(R, K // 32)).astype(np.uint16)
    wq = (q * np.repeat(sb.view(np.float16).astype(np.float64), 32, axis=1)).astype(np.float32)
    u2, s2 = C.quantize(wq)
    np.testing.assert_array_equal(s2, sb)
    np.testing.assert_array_equal(u2 - 8, q)
    np.testing.assert_array_equal(C.dequant(C.pack_codes(u2), s2, K), wq.astype(np.float64))
    uz, sz = C.quantize(np.zeros((2, 128), np.float32))
    assert np.all(sz == 0) and np.all(uz == 8)


def test_fp4_dequant_hand_worked_rows():
    """MXFP4: code 7 (6.0) at element 37 with scale byte 125 (1/4), code 9
    (-0.5) at element 100 with byte 130 (8).  NVFP4: the same codes, E4M3
    bytes 0x38 (1.0) on block 2 and 0x46 (3.5) on block 6, matrix scale 0.5."""
    u = np.zeros((1, 128), np.uint8)
    u[0, 37], u[0, 100] = 7, 9
    w = C.dequant(C.pack_codes(u), np.array([[127, 125, 127, 130]], np.uint8), 128, fmt=1)[0]
    want = np.zeros(128)
    want[37], want[100] = 1.5, -4.0
    assert np.array_equal(w, want)
    s = np.zeros((1, 8), np.uint8)
    s[0, 2], s[0, 6] = 0x38, 0x46
    w = C.dequant(C.pack_codes(u), s, 128, fmt=2, ts=0.5)[0]
    want[37], want[100] = 6.0 * 1.0 * 0.5, -0.5 * 3.5 * 0.5
    assert np.array_equal(w, want)


# ------------------------------------------------------------------ router and selection


def test_router_one_hot_and_integer_exact():
    lay = tiny()
    for k0 in (0, 7, 255):
        x = np.zeros(256, np.uint16)
        x[k0] = 0x3F80
        np.testing.assert_array_equal(C.router_logits(lay, x), lay["router_w"][:, k0].astype(np.float64))
    rng = np.random.default_rng(3)
    W = rng.integers(-50, 51, size=(16, 256)).astype(np.float32)
    xi = rng.integers(-8, 9, size=256)
    b = rng.integers(-5, 6, size=16).astype(np.float32)
    xb = C.f64_to_bf16_bits(xi.astype(np.float64))  # small integers are exact in bf16
    lay2 = dict(lay, router_w=W, router_b=b)
    want = [sum(int(W[e, k]) * int(xi[k]) for k in range(256)) + int(b[e]) for e in range(16)]
    np.testing.assert_array_equal(C.router_logits(lay2, xb), want)


def test_route_brute_force_closed_forms_and_ties():
    for seed in range(1, 6):
        lay = tiny(seed=seed)
        l = C.router_logits(lay, tiny_x(lay, seed=seed))
        S, w = C.route(l, 2)
        best = max(combinations(range(16), 2), key=lambda c: l[c[0]] + l[c[1]])
        assert sorted(S.tolist()) == sorted(best) and math.isclose(w.sum(), 1.0, rel_tol=1e-15) and w[0] >= w[1]
    l = np.array([0.0, math.log(2.0), math.log(5.0)])
    S, w = C.route(l, 3, norm_topk=False)
    assert S.tolist() == [2, 1, 0]
    np.testing.assert_allclose(w, [5 / 8, 2 / 8, 1 / 8], rtol=1e-15)
    S, w = C.route(l + 123.0, 2)
    np.testing.assert_allclose(w, [5 / 7, 2 / 7], rtol=1e-14)
    assert C.route(np.array([0.1, 0.3, 0.3, 0.3]), 4)[0].tolist() == [1, 2, 3, 0]
    l = np.random.default_rng(21).standard_normal(16) * 2.0 ** 20   # all but one probability underflow
    S, w = C.route(l, 4)
    assert np.all(np.diff(l[S]) < 0) and w.tolist() == [1.0, 0.0, 0.0, 0.0]


# ------------------------------------------------------------------ layer


@pytest.mark.parametrize("cfg", [synth.TINY, synth.TINY_SHARED, synth.TINY_FP4, synth.TINY_NV],
                         ids=["int4", "shared", "mxfp4", "nvfp4"])
def test_sparse_equals_all_experts_then_mask_bit_exact(cfg):
    lay = tiny(cfg, 2)
    x = tiny_x(lay, cfg, 2)
    out = C.moe_forward(lay, x, cfg.k)
    ym, read_all = C.moe_forward_masked(lay, x, cfg.k)
    assert np.array_equal(out["y"], ym)
    E, d, f, k, ns = cfg.E, cfg.d, cfg.f, cfg.k, int("shared_gate_q" in lay)
    assert out["weights_read"] == E * d + (k + ns) * 3 * d * f
    assert read_all == E * d + (E + ns) * 3 * d * f


def _single_expert_layer():
    g = {ln[0]: ln[1:] for ln in golden_lines("swiglu_single_expert.txt")}
    d = f = 128
    k0 = int(g["k0"][0])
    i = np.arange(f)
    ug = np.full((f, d), 8)
    uu = np.full((f, d), 8)
    ug[:, k0] = 8 + np.where(i % 3 == 0, 1, np.where(i % 3 == 1, -1, 0))
    uu[:, k0] = 8 + np.where(i < 64, 1, -1)
    ud = np.full((d, f), 8)
    ud[np.arange(d), np.arange(d)] = 9
    one = np.full((f, d // 32), 0x3C00, np.uint16)
    lay = dict(router_w=np.ones((1, d), np.float32), router_b=None,
               gate_q=C.pack_codes(ug)[None], gate_s=one[None], up_q=C.pack_codes(uu)[None], up_s=one[None],
               down_q=C.pack_codes(ud)[None], down_s=one[None])
    x = np.zeros(d, np.uint16)
    x[k0] = 0x3F80
    sp, sm = float(g["silu_plus1"][0]), float(g["silu_minus1"][0])
    want = np.where(i % 3 == 0, sp, np.where(i % 3 == 1, sm, 0.0)) * np.where(i < 64, 1.0, -1.0)
    return lay, x, want


def test_single_expert_is_the_hand_worked_swiglu_and_shared_alone_too():
    lay, x, want = _single_expert_layer()
    out = C.moe_forward(lay, x, 1)
    assert out["idx"].tolist() == [0] and out["w"].tolist() == [1.0]
    np.testing.assert_allclose(out["y"], want, rtol=1e-15, atol=0)
    # two routed experts that read as exact zeros, the hand-worked one shared
    z = {n: np.stack([lay[n][0]] * 2) for n in ("gate_q", "up_q", "down_q")}
    zero_q = C.pack_codes(np.full((128, 128), 8))
    sh = dict(router_w=np.ones((2, 128), np.float32), router_b=None,
              gate_q=np.stack([zero_q] * 2), gate_s=np.stack([lay["gate_s"][0]] * 2),
              up_q=np.stack([zero_q] * 2), up_s=np.stack([lay["up_s"][0]] * 2),
              down_q=np.stack([zero_q] * 2), down_s=np.stack([lay["down_s"][0]] * 2),
              **{"shared_" + n: lay[n][0] for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")})
    del z
    np.testing.assert_allclose(C.moe_forward(sh, x, 1)["y"], want, rtol=1e-15, atol=0)
    np.testing.assert_allclose(C.moe_forward_masked(sh, x, 1)[0], want, rtol=1e-15, atol=0)


def test_all_experts_is_the_softmax_mixture_and_on_set():
    lay = tiny(seed=5)
    x = tiny_x(lay, seed=5)
    out = C.moe_forward(lay, x, 16)
    p = np.exp(out["logits"] - out["logits"].max())
    p /= p.sum()
    np.testing.assert_allclose(out["w"], p[out["idx"]], rtol=1e-14)
    # the same set given in another order: the same y; a set's weights: p over the set
    o = C.moe_forward_on_set(lay, x, out["idx"][::-1])
    np.testing.assert_allclose(o["y"], out["y"], rtol=0, atol=1e-15 * np.abs(out["y"]).max())
    S = np.array([11, 3, 7])
    o = C.moe_forward_on_set(lay, x, S, False)
    np.testing.assert_allclose(o["w"], p[S], rtol=1e-14)


def test_scale_linearity_and_permutation_equivariance():
    lay = tiny(seed=6)
    x = tiny_x(lay, seed=6)
    y = C.moe_forward(lay, x, 2)["y"]
    for name in ("down_s", "up_s"):
        s2 = C.f64_to_f16_bits(C.f16_to_f64(lay[name]) * 2)
        assert np.array_equal(C.moe_forward(dict(lay, **{name: s2}), x, 2)["y"], 2 * y)
    perm = np.random.default_rng(7).permutation(16)
    lp = {n: (v[perm] if n in ("router_w", "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s") else v)
          for n, v in lay.items()}
    out, outp = C.moe_forward(lay, x, 2), C.moe_forward(lp, x, 2)
    assert sorted(perm[outp["idx"]].tolist()) == sorted(out["idx"].tolist())
    np.testing.assert_allclose(outp["y"], out["y"], rtol=0, atol=1e-15 * np.abs(out["y"]).max())


# ------------------------------------------------------------------ stack


def _one_entry_layer(gate, up, down):
    d = f = 128
    codes = {n: np.full(shape, 8) for n, shape in (("g", (f, d)), ("u", (f, d)), ("d", (d, f)))}
    scales = {n: np.full((128, 4), 0x3C00, np.uint16) for n in ("g", "u", "d")}
    for n, ents, sc in (("g", gate, 0x3000), ("u", up, 0x3000), ("d", down, 0x3C00)):
        for r, c, u in ents:
            codes[n][r, c] = u
            scales[n][r, c // 32] = sc
    return dict(router_w=np.ones((1, d), np.float32), router_b=None,
                gate_q=C.pack_codes(codes["g"])[None], gate_s=scales["g"][None],
                up_q=C.pack_codes(codes["u"])[None], up_s=scales["u"][None],
                down_q=C.pack_codes(codes["d"])[None], down_s=scales["d"][None])


def test_stack_two_layers_hand_worked():
    g = {ln[0]: float(ln[1]) for ln in golden_lines("stack_two_layers.txt")}
    k0 = int(g["k0"])
    A = _one_entry_layer(gate=[(0, k0, 9)], up=[(0, k0, 9)], down=[(9, 0, 9)])
    B = _one_entry_layer(gate=[(0, 9, 9)], up=[(0, k0, 9)], down=[(k0, 0, 7)])
    x0 = np.zeros(128, np.uint16)
    x0[k0] = 0x3F80
    out = C.stack_forward([A, B], x0, 1, 1e-6)
    x1, x2 = C.bf16_to_f64(out["xs"][0]), C.bf16_to_f64(out["xs"][1])
    assert x1[k0] == g["x1_k0"] and np.count_nonzero(x1) == 1
    assert x2[k0] == g["x2_k0"] and x2[9] == g["x2_9"] and np.count_nonzero(x2) == 2
    yA, yB = out["ys"]
    assert yA[9] == np.float32(g["yA_9"]) and np.count_nonzero(yA) == 1
    assert yB[k0] == np.float32(g["yB_k0"]) and np.count_nonzero(yB) == 1
    r = out["r"]
    assert r[k0] == np.float32(g["r2_k0"]) and r[9] == np.float32(g["r2_9"]) and np.count_nonzero(r) == 2


def test_rmsnorm_closed_forms_and_zero_layers_keep_the_residual():
    for c in (0.5, -3.0, 1e-3):
        x = C.rmsnorm_bf16(np.full(64, c, np.float32), 1e-6)
        want = C.f64_to_bf16_bits(np.float64(np.float32(c)) / math.sqrt(np.float64(np.float32(c)) ** 2 + 1e-6))
        assert np.all(x == want)
    lay = tiny(seed=9)
    Z = dict(lay, gate_s=np.zeros_like(lay["gate_s"]), down_s=np.zeros_like(lay["down_s"]))
    x0 = synth.draw_x(synth.TINY, 9, 0, 0, 0)
    out = C.stack_forward([Z, Z, Z], x0, 2)
    np.testing.assert_array_equal(out["r"], C.bf16_to_f64(x0).astype(np.float32))
    assert all(np.all(y == 0) for y in out["ys"])


def test_group_by_expert_hand_example():
    off, order, active = C.group_by_expert(np.array([[2, 0], [2, 3], [0, 2]]), 5)
    assert off.tolist() == [0, 2, 2, 5, 6, 6] and order.tolist() == [1, 4, 0, 2, 5, 3]
    assert active.tolist() == [0, 2, 3]


# ------------------------------------------------------------------ LM head


def test_lmhead_v16_hand_worked_with_tie_and_planted_row():
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
        s[v, 0] = C.f64_to_f16_bits([float(sv)])[0]
        z_want[v] = float(z)
    x = np.zeros((1, d), np.uint16)
    x[0, 0], x[0, 1] = 0x3F80, 0x4000
    tok, zmax, z = C.lmhead_argmax(C.pack_codes(u), s, x)
    np.testing.assert_array_equal(z[0], z_want)
    assert tok[0] == token and zmax[0] == 21.0

    q, s = synth.int4_matrix(4096, 256, synth.key(11, "lmhead-test"), 0.02)
    x = synth.bf16(256, synth.key(11, "hidden-test"))
    xf = C.bf16_to_f64(x)
    uu = C.unpack_codes(q, 256)
    uu[1234] = np.where(xf >= 0, 15, 1)
    q2 = q.copy()
    q2[1234] = C.pack_codes(uu[1234][None])[0]
    s2 = s.copy()
    s2[1234] = C.f64_to_f16_bits(np.full(8, 0.05))
    tok, zmax, _ = C.lmhead_argmax(q2, s2, x[None])
    assert tok[0] == 1234
    assert np.isclose(zmax[0], C.f16_to_f64(s2[1234, :1])[0] * 7 * np.abs(xf).sum(), rtol=1e-12)


# ------------------------------------------------------------------ the two oracles


@pytest.mark.parametrize("cfg", [synth.TINY, synth.TINY_SHARED, synth.TINY_FP4, synth.TINY_NV],
                         ids=["int4", "shared", "mxfp4", "nvfp4"])
def test_agrees_with_the_numpy_oracle(cfg):
    """The C++ and numpy oracles, written independently, on seeded layers:
    the same chosen sets, weights and outputs to fp64 rounding."""
    for seed in (1, 3):
        lay = tiny(cfg, seed)
        x = tiny_x(lay, cfg, seed)
        a, b = M.moe_forward(M.Layer.from_dict(lay), x, cfg.k), C.moe_forward(lay, x, cfg.k)
        assert a["idx"].tolist() == b["idx"].tolist()
        np.testing.assert_allclose(b["w"], a["w"], rtol=1e-13)
        np.testing.assert_allclose(b["y"], a["y"], rtol=0, atol=1e-13 * np.abs(a["y"]).max())


def test_stack_and_lmhead_agree_with_the_numpy_oracle():
    from oracle import lmhead as H
    lays = [synth.make_layer(synth.TINY, 4, l) for l in range(3)]
    x0 = synth.draw_x(synth.TINY, 4, 0, 0, 0)
    a = M.stack_forward([M.Layer.from_dict(l) for l in lays], x0, 2)
    b = C.stack_forward(lays, x0, 2)
    for l in range(3):
        assert sorted(a["idx"][l].tolist()) == sorted(b["idx"][l].tolist())
    np.testing.assert_allclose(b["r"], a["r"], rtol=0, atol=1e-5 * np.abs(a["r"]).max())
    q, s = synth.int4_matrix(2048, 256, synth.key(13, "lm-x"), 0.02)
    X = np.stack([synth.bf16(256, synth.key(13, "h", b)) for b in range(3)])
    t1, z1, _ = H.lmhead_argmax(q, s, X)
    t2, z2, _ = C.lmhead_argmax(q, s, X)
    assert t1.tolist() == t2.tolist()
    np.testing.assert_allclose(z2, z1, rtol=1e-13)


def test_threads_do_not_change_results():
    lay = synth.make_layer(synth.TINY, 2)
    x = tiny_x(lay, seed=2)
    n0 = C.get_threads()
    try:
        C.set_threads(1)
        a = C.moe_forward(lay, x, 2)
        C.set_threads(max(2, C.hw_threads()))
        b = C.moe_forward(lay, x, 2)
    finally:
        C.set_threads(n0)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["idx"], b["idx"])
    assert C.hw_threads() >= 1
