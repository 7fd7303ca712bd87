"""Pins of the MoE-layer oracle: closed forms, brute force over tiny inputs,
a hand-worked single-expert case and invariants.  None of these compute the
expected value with the function under test."""
import math

import numpy as np
import pytest

import synth
from conftest import golden_lines
from oracle import formats as F
from oracle import moe as M


def tiny_layer(seed=1):
    return M.Layer.from_dict(synth.make_layer(synth.TINY, seed))


def tiny_x(layer, seed=1, token=0):
    from oracle.inputs import pick_token
    x, _ = pick_token(layer, synth.TINY.k, synth.TINY.margin,
                      lambda a: synth.draw_x(synth.TINY, seed, 0, token, a))
    return x


def test_router_one_hot_column():
    L = tiny_layer()
    for k0 in (0, 7, 255):
        x = np.zeros(L.d)
        x[k0] = 1.0
        np.testing.assert_array_equal(M.router_logits(L, x), L.router_w[:, k0].astype(np.float64))


def test_router_integer_exact():
    rng = np.random.default_rng(3)
    E, d = 16, 256
    W = rng.integers(-50, 51, size=(E, d)).astype(np.float32)
    xi = rng.integers(-8, 9, size=d)
    b = rng.integers(-5, 6, size=E).astype(np.float32)
    L = M.Layer(W, b, *[None] * 6)
    want = [sum(int(W[e, k]) * int(xi[k]) for k in range(d)) + int(b[e]) for e in range(E)]
    np.testing.assert_array_equal(M.router_logits(L, xi.astype(np.float64)), want)


def test_topk_equals_best_subset_bruteforce():
    for seed in range(1, 6):
        L = tiny_layer(seed)
        x = F.bf16_to_f64(tiny_x(L, seed))
        l = M.router_logits(L, x)
        S, w = M.route(l, 2)
        assert sorted(S.tolist()) == sorted(M.best_subset_bruteforce(l, 2).tolist())
        assert math.isclose(w.sum(), 1.0, rel_tol=1e-15)
        assert w[0] >= w[1]


def test_topk_where_probabilities_underflow():
    """Logits spread over 2^20: all but the largest softmax probability
    underflow to 0 in fp64, yet the chosen set is still the k largest
    logits (the brute-force best subset), in descending order."""
    rng = np.random.default_rng(21)
    l = rng.standard_normal(16) * 2.0 ** 20
    p = M.softmax(l)
    assert np.count_nonzero(p) == 1
    S, w = M.route(l, 4)
    assert sorted(S.tolist()) == sorted(M.best_subset_bruteforce(l, 4).tolist())
    assert np.all(np.diff(l[S]) < 0)
    assert w.tolist() == [1.0, 0.0, 0.0, 0.0]


def test_topk_tie_lower_index_first():
    p = np.array([0.1, 0.3, 0.3, 0.3])
    assert M.select_topk(p, 1).tolist() == [1]
    assert M.select_topk(p, 2).tolist() == [1, 2]
    assert M.select_topk(p, 4).tolist() == [1, 2, 3, 0]


def test_softmax_shift_invariance_and_closed_form():
    l = np.array([0.0, math.log(2.0), math.log(5.0)])
    np.testing.assert_allclose(M.softmax(l), [1 / 8, 2 / 8, 5 / 8], rtol=1e-15)
    np.testing.assert_allclose(M.softmax(l + 123.0), [1 / 8, 2 / 8, 5 / 8], rtol=1e-14)


def test_norm_topk_off_keeps_softmax_values():
    l = np.array([0.0, math.log(2.0), math.log(5.0)])
    S, w = M.route(l, 2, norm_topk=False)
    assert S.tolist() == [2, 1]
    np.testing.assert_allclose(w, [5 / 8, 2 / 8], rtol=1e-15)
    S, w = M.route(l, 2, norm_topk=True)
    np.testing.assert_allclose(w, [5 / 7, 2 / 7], rtol=1e-15)


def test_margin_values():
    l = np.array([0.5, 0.2, 0.9, 0.25])
    assert math.isclose(M.topk_margin(l, 1), 0.4)
    assert math.isclose(M.topk_margin(l, 2), 0.25)
    assert math.isclose(M.topk_margin(l, 3), 0.05)
    assert M.topk_margin(l, 4) == float("inf")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_sparse_equals_all_experts_then_mask_bit_exact(seed):
    L = tiny_layer(seed)
    x = tiny_x(L, seed)
    y_sparse = M.moe_forward(L, x, 2)["y"]
    y_masked = M.moe_forward_masked(L, x, 2)
    assert np.array_equal(y_sparse, y_masked)


@pytest.mark.parametrize("norm", [True, False])
def test_sparse_matches_independent_dense_einsum(norm):
    L = tiny_layer(4)
    x = tiny_x(L, 4)
    y = M.moe_forward(L, x, 2, norm)["y"]
    y2 = M.moe_forward_dense_einsum(L, x, 2, norm)
    np.testing.assert_allclose(y, y2, rtol=0, atol=1e-13 * np.abs(y2).max())


def test_active_weight_count():
    L = tiny_layer()
    x = tiny_x(L)
    L.weights_read = 0
    M.moe_forward(L, x, 2)
    E, d, f, k = 16, 256, 128, 2
    assert L.weights_read == E * d + k * 3 * d * f == M.active_weights(E, d, f, k)
    L.weights_read = 0
    M.moe_forward_masked(L, x, 2)
    assert L.weights_read == E * d + E * 3 * d * f
    # the flagship layer shape: 256 experts, top-8, d=2048, f=512
    assert M.active_weights(256, 2048, 512, 8) == 524288 + 25165824


def test_all_experts_selected_is_the_softmax_mixture():
    L = tiny_layer(5)
    x = tiny_x(L, 5)
    out = M.moe_forward(L, x, 16)
    p = np.exp(out["logits"] - out["logits"].max())
    p /= p.sum()
    np.testing.assert_allclose(out["w"], p[out["idx"]], rtol=1e-14)
    xs = F.bf16_to_f64(x)
    y = sum(p[e] * M.expert_forward(*L.expert(e), xs) for e in range(16))
    np.testing.assert_allclose(out["y"], y, rtol=0, atol=1e-14 * np.abs(y).max())


def _single_expert_layer():
    g = {ln[0]: ln[1:] for ln in golden_lines("swiglu_single_expert.txt")}
    d = f = 128
    k0 = int(g["k0"][0])
    ug = np.full((f, d), 8)
    uu = np.full((f, d), 8)
    i = np.arange(f)
    ug[:, k0] = 8 + np.where(i % 3 == 0, 1, np.where(i % 3 == 1, -1, 0))
    uu[:, k0] = 8 + np.where(i < 64, 1, -1)
    ud = np.full((d, f), 8)
    ud[np.arange(d), np.arange(d)] = 9
    one = np.full((f, d // 32), 0x3C00, np.uint16)
    L = M.Layer(np.ones((1, d), np.float32), None,
                F.pack_codes(ug)[None], one[None], F.pack_codes(uu)[None], one[None],
                F.pack_codes(ud)[None], np.full((d, f // 32), 0x3C00, np.uint16)[None])
    x = np.zeros(d, np.uint16)
    x[k0] = 0x3F80
    return L, x, g, i


def test_single_expert_is_plain_swiglu_mlp_hand_worked():
    L, x, g, i = _single_expert_layer()
    sp, sm = float(g["silu_plus1"][0]), float(g["silu_minus1"][0])
    want = np.where(i % 3 == 0, sp, np.where(i % 3 == 1, sm, 0.0)) * np.where(i < 64, 1.0, -1.0)
    out = M.moe_forward(L, x, 1)
    assert out["idx"].tolist() == [0] and out["w"].tolist() == [1.0]
    np.testing.assert_allclose(out["y"], want, rtol=1e-15, atol=0)


def test_scale_linearity_exact():
    """Doubling every down (or every up) scale doubles y exactly: binary16
    scales times 2 are exact, and so is every product and sum scaled by 2."""
    L = tiny_layer(6)
    x = tiny_x(L, 6)
    y = M.moe_forward(L, x, 2)["y"]
    for name in ("down_s", "up_s"):
        L2 = tiny_layer(6)
        s = getattr(L2, name)
        setattr(L2, name, F.f64_to_f16_bits(F.f16_to_f64(s) * 2))
        assert np.array_equal(M.moe_forward(L2, x, 2)["y"], 2 * y)


def test_expert_permutation_equivariance():
    L = tiny_layer(7)
    x = tiny_x(L, 7)
    out = M.moe_forward(L, x, 2)
    perm = np.random.default_rng(7).permutation(16)
    Lp = M.Layer(L.router_w[perm], None, L.gate_q[perm], L.gate_s[perm], L.up_q[perm], L.up_s[perm],
                 L.down_q[perm], L.down_s[perm])
    outp = M.moe_forward(Lp, x, 2)
    assert sorted(perm[outp["idx"]].tolist()) == sorted(out["idx"].tolist())
    np.testing.assert_allclose(outp["y"], out["y"], rtol=0, atol=1e-15 * np.abs(out["y"]).max())


def test_rmsnorm_closed_forms():
    eps = 1e-6
    for c in (0.5, -3.0, 1e-3):
        x = M.rmsnorm_bf16(np.full(64, c), eps)
        assert np.all(x == F.f64_to_bf16_bits(c / math.sqrt(c * c + eps)))
    r = np.random.default_rng(8).standard_normal(2048) * 3
    xh = r / np.sqrt(np.mean(r * r) + eps)
    m = np.mean(r * r)
    assert math.isclose(np.mean(xh * xh), m / (m + eps), rel_tol=1e-12)
    got = F.bf16_to_f64(M.rmsnorm_bf16(r, eps))
    assert np.all(np.abs(got - xh) <= np.abs(xh) * 2.0 ** -8)


def test_stack_of_zero_experts_keeps_the_residual():
    """Layers whose expert scales are all zero output y = 0, so the residual
    stream is unchanged through the whole stack."""
    L = tiny_layer(9)
    Z = M.Layer(L.router_w, None, L.gate_q, np.zeros_like(L.gate_s), L.up_q, L.up_s,
                L.down_q, np.zeros_like(L.down_s))
    x0 = synth.draw_x(synth.TINY, 9, 0, 0, 0)
    out = M.stack_forward([Z, Z, Z], x0, 2)
    np.testing.assert_array_equal(out["r"], F.bf16_to_f64(x0).astype(np.float32))
    assert all(np.all(y == 0) for y in out["ys"])


def _one_entry_layer(gate, up, down):
    """E = 1, d = f = 128, every weight 0 except gate/up entries (row, col,
    code) with a binary16 scale of 1/8 on their group and down entries with
    scale 1."""
    d = f = 128
    codes = {n: np.full(shape, 8) for n, shape in (("g", (f, d)), ("u", (f, d)), ("d", (d, f)))}
    scales = {n: np.full((shape[0], shape[1] // 32), 0x3C00, np.uint16)
              for n, shape in (("g", (f, d)), ("u", (f, d)), ("d", (d, f)))}
    for n, ents, sc in (("g", gate, 0x3000), ("u", up, 0x3000), ("d", down, 0x3C00)):
        for r, c, u in ents:
            codes[n][r, c] = u
            scales[n][r, c // 32] = sc
    return M.Layer(np.ones((1, d), np.float32), None,
                   F.pack_codes(codes["g"])[None], scales["g"][None], F.pack_codes(codes["u"])[None],
                   scales["u"][None], F.pack_codes(codes["d"])[None], scales["d"][None])


def test_stack_two_layers_hand_worked():
    """The pre-norm residual stack of two one-expert layers against the
    values worked by hand in golden/stack_two_layers.txt: the bf16 pre-norm
    of every layer, each layer's output and the fp32 residual after both.
    Feeding the un-normalized r_l to a layer, or adding y twice, fails it."""
    g = {ln[0]: float(ln[1]) for ln in golden_lines("stack_two_layers.txt")}
    k0 = int(g["k0"])
    A = _one_entry_layer(gate=[(0, k0, 9)], up=[(0, k0, 9)], down=[(9, 0, 9)])
    B = _one_entry_layer(gate=[(0, 9, 9)], up=[(0, k0, 9)], down=[(k0, 0, 7)])
    x0 = np.zeros(128, np.uint16)
    x0[k0] = 0x3F80  # bf16 1.0
    out = M.stack_forward([A, B], x0, 1, 1e-6)
    x1, x2 = F.bf16_to_f64(out["xs"][0]), F.bf16_to_f64(out["xs"][1])
    assert x1[k0] == g["x1_k0"] and np.count_nonzero(x1) == 1
    assert x2[k0] == g["x2_k0"] and x2[9] == g["x2_9"] and np.count_nonzero(x2) == 2
    yA, yB = out["ys"]
    assert yA.dtype == np.float32 and yA[9] == np.float32(g["yA_9"]) and np.count_nonzero(yA) == 1
    assert yB[k0] == np.float32(g["yB_k0"]) and np.count_nonzero(yB) == 1
    r = out["r"]
    assert r.dtype == np.float32
    assert r[k0] == np.float32(g["r2_k0"]) and r[9] == np.float32(g["r2_9"]) and np.count_nonzero(r) == 2


def test_forward_on_given_set():
    """moe_forward_on_set: on the selected set it is moe_forward exactly; on
    any set of identical experts it reduces to one expert's output times the
    sum of the weights (1 with renormalization, sum of the softmax values
    without); the order in which S is given does not matter."""
    L = tiny_layer(6)
    x = tiny_x(L, 6)
    ref = M.moe_forward(L, x, 2)
    got = M.moe_forward_on_set(L, x, ref["idx"])
    assert np.array_equal(got["y"], ref["y"]) and np.array_equal(got["w"], ref["w"])
    assert np.array_equal(M.moe_forward_on_set(L, x, ref["idx"][::-1])["y"], ref["y"])

    # every expert a copy of expert 0: y over any set is o_0 * sum(w)
    t = synth.make_layer(synth.TINY, 6)
    for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        t[n] = np.repeat(t[n][:1], t[n].shape[0], axis=0)
    C = M.Layer.from_dict(t)
    o0 = M.expert_forward(*C.expert(0), F.bf16_to_f64(x))
    S = np.array([11, 3, 7])      # not the top-3 in general
    y1 = M.moe_forward_on_set(C, x, S, True)["y"]
    np.testing.assert_allclose(y1, o0, rtol=0, atol=1e-14 * np.abs(o0).max())
    p = M.softmax(M.router_logits(C, F.bf16_to_f64(x)))
    y0 = M.moe_forward_on_set(C, x, S, False)["y"]
    np.testing.assert_allclose(y0, o0 * p[S].sum(), rtol=0, atol=1e-14 * np.abs(o0).max())


def test_group_by_expert_hand_example_and_invariants():
    """Tokens (0: experts 2,0), (1: 2,3), (2: 0,2) with E = 5: expert 0 owns
    assignments 1 and 4, expert 2 owns 0, 2 and 5, expert 3 owns 3."""
    off, order, active = M.group_by_expert(np.array([[2, 0], [2, 3], [0, 2]]), 5)
    assert off.tolist() == [0, 2, 2, 5, 6, 6]
    assert order.tolist() == [1, 4, 0, 2, 5, 3]
    assert active.tolist() == [0, 2, 3]
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(40, 6, replace=False) for _ in range(33)])
    off, order, active = M.group_by_expert(idx, 40)
    assert sorted(order.tolist()) == list(range(idx.size))          # each assignment once
    assert np.array_equal(np.diff(off), np.bincount(idx.ravel(), minlength=40))
    for e in range(40):
        seg = order[off[e]:off[e + 1]]
        assert np.all(idx.ravel()[seg] == e) and np.all(np.diff(seg) > 0)
    assert active.tolist() == [e for e in range(40) if off[e + 1] > off[e]]


# ------------------------------------------------------------------ shared expert


def _shared_alone_layer():
    """Routed experts that read as exact zeros (code 8, scale 1) and the
    hand-worked single expert as the shared one."""
    L1, x, g, i = _single_expert_layer()
    d = f = 128
    zeros_q = F.pack_codes(np.full((f, d), 8))
    one = np.full((f, d // 32), 0x3C00, np.uint16)
    E = 2
    L = M.Layer(np.ones((E, d), np.float32), None,
                np.stack([zeros_q] * E), np.stack([one] * E), np.stack([zeros_q] * E), np.stack([one] * E),
                np.stack([zeros_q] * E), np.stack([one] * E),
                shared=(L1.gate_q[0], L1.gate_s[0], L1.up_q[0], L1.up_s[0], L1.down_q[0], L1.down_s[0]))
    return L, x, g, i


def test_shared_expert_alone_is_the_hand_worked_swiglu():
    """With routed experts of zero weight the output is the shared expert's:
    the hand-worked SwiGLU values, added with weight 1."""
    L, x, g, i = _shared_alone_layer()
    sp, sm = float(g["silu_plus1"][0]), float(g["silu_minus1"][0])
    want = np.where(i % 3 == 0, sp, np.where(i % 3 == 1, sm, 0.0)) * np.where(i < 64, 1.0, -1.0)
    out = M.moe_forward(L, x, 1)
    np.testing.assert_allclose(out["y"], want, rtol=1e-15, atol=0)
    np.testing.assert_allclose(M.moe_forward_masked(L, x, 1), want, rtol=1e-15, atol=0)


def test_shared_expert_weight_one_and_routing_untouched():
    """The shared expert changes neither the chosen set nor its weights, and
    enters with weight 1: doubling its down scales adds its output once more."""
    lay = synth.make_layer(synth.TINY_SHARED, 3)
    Ls = M.Layer.from_dict(lay)
    L0 = M.Layer.from_dict({k: v for k, v in lay.items() if not k.startswith("shared")})
    x = tiny_x(L0, 3)
    a, b = M.moe_forward(Ls, x, 2), M.moe_forward(L0, x, 2)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["w"], b["w"])
    assert np.array_equal(a["logits"], b["logits"])
    lay2 = dict(lay, shared_down_s=F.f64_to_f16_bits(F.f16_to_f64(lay["shared_down_s"]) * 2))
    c = M.moe_forward(M.Layer.from_dict(lay2), x, 2)
    s = a["y"] - b["y"]
    assert np.abs(s).max() > 1e-3
    np.testing.assert_allclose(c["y"] - a["y"], s, rtol=0, atol=1e-15 * np.abs(a["y"]).max())


@pytest.mark.parametrize("seed", [1, 2])
def test_shared_sparse_equals_all_experts_then_mask_and_dense(seed):
    lay = synth.make_layer(synth.TINY_SHARED, seed)
    L = M.Layer.from_dict(lay)
    x = tiny_x(M.Layer.from_dict({k: v for k, v in lay.items() if not k.startswith("shared")}), seed)
    y = M.moe_forward(L, x, 2)["y"]
    assert np.array_equal(y, M.moe_forward_masked(M.Layer.from_dict(lay), x, 2))
    yd = M.moe_forward_dense_einsum(M.Layer.from_dict(lay), x, 2)
    np.testing.assert_allclose(y, yd, rtol=0, atol=1e-13 * np.abs(y).max())


def test_shared_active_weight_count():
    lay = synth.make_layer(synth.TINY_SHARED, 1)
    L = M.Layer.from_dict(lay)
    x = tiny_x(L, 1)
    L.weights_read = 0
    M.moe_forward(L, x, 2)
    E, d, f, k = 16, 256, 128, 2
    assert L.weights_read == E * d + (k + 1) * 3 * d * f == M.active_weights(E, d, f, k, 1)
    # the pages' layer: 256 routed experts, top-6 plus one shared, d=2048, f=512
    assert M.active_weights(256, 2048, 512, 6, 1) == 524288 + 7 * 3 * 2048 * 512


# ------------------------------------------------------------------ MXFP4 layers


def tiny_fp4_layer(seed=1):
    return M.Layer.from_dict(synth.make_layer(synth.TINY_FP4, seed))


@pytest.mark.parametrize("seed", [1, 2])
def test_fp4_sparse_equals_mask_and_dense(seed):
    """An MXFP4 layer: the sparse step equals all experts then mask (bit for
    bit) and the independent dense einsum."""
    L = tiny_fp4_layer(seed)
    x = tiny_x(L, seed)
    y = M.moe_forward(L, x, 2)["y"]
    assert np.array_equal(y, M.moe_forward_masked(L, x, 2))
    y2 = M.moe_forward_dense_einsum(L, x, 2)
    np.testing.assert_allclose(y, y2, rtol=0, atol=1e-13 * np.abs(y2).max())


def test_fp4_layer_reads_e2m1_values_times_power_of_two_scales():
    """The MXFP4 layer's expert matrices are exactly the E2M1 table values
    (tests/golden/fp4_e2m1.txt) times 2^(b-127): every weight divided by its
    block's scale is one of the 15 distinct table values; and raising every
    down scale byte by one doubles y exactly."""
    L = tiny_fp4_layer(3)
    table = {float(r[1]) for r in golden_lines("fp4_e2m1.txt")}
    Wg, _, Wd = L.expert(0)
    s = 2.0 ** (L.gate_s[0].astype(np.float64) - 127.0)
    v = Wg.reshape(Wg.shape[0], -1, 32) / s[..., None]
    assert set(np.unique(v).tolist()) <= table
    x = tiny_x(L, 3)
    y = M.moe_forward(L, x, 2)["y"]
    L2 = tiny_fp4_layer(3)
    L2.down_s = (L2.down_s.astype(np.int64) + 1).astype(np.uint8)
    assert np.array_equal(M.moe_forward(L2, x, 2)["y"], 2 * y)


# ------------------------------------------------------------------ NVFP4 layers


@pytest.mark.parametrize("seed", [1, 2])
def test_nvfp4_sparse_equals_mask_and_dense(seed):
    """An NVFP4 layer (E4M3 per 16, fp32 per matrix): sparse == all experts
    then mask (bit for bit) == the independent dense einsum."""
    L = M.Layer.from_dict(synth.make_layer(synth.TINY_NV, seed))
    x = tiny_x(L, seed)
    y = M.moe_forward(L, x, 2)["y"]
    assert np.array_equal(y, M.moe_forward_masked(L, x, 2))
    y2 = M.moe_forward_dense_einsum(L, x, 2)
    np.testing.assert_allclose(y, y2, rtol=0, atol=1e-13 * np.abs(y2).max())


def test_nvfp4_tensor_scale_is_linear_and_weights_are_table_values():
    """Every NVFP4 weight is an E2M1 table value times an E4M3 value times
    the matrix's fp32 scale, and doubling every down tensor scale doubles y
    exactly."""
    lay = synth.make_layer(synth.TINY_NV, 3)
    L = M.Layer.from_dict(lay)
    table = {float(r[1]) for r in golden_lines("fp4_e2m1.txt")}
    Wg, _, _ = L.expert(1)
    s = F.e4m3_to_f64(lay["gate_s"][1]) * np.float64(lay["gate_ts"][1])
    v = Wg.reshape(Wg.shape[0], -1, 16) / np.where(s == 0, 1, s)[..., None]
    assert set(np.unique(v).tolist()) <= table
    x = tiny_x(L, 3)
    y = M.moe_forward(L, x, 2)["y"]
    L2 = M.Layer.from_dict(dict(lay, down_ts=(lay["down_ts"] * 2).astype(np.float32)))
    assert np.array_equal(M.moe_forward(L2, x, 2)["y"], 2 * y)
