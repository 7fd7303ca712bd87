"""CPU check of the int4 x bf16 dot-product identity the kernels rely on.

The masks, shifts, magic constant, activation scaling and correction
coefficients are read out of the kernel header (device_common.h) and
emulated bit for bit in numpy, so a wrong constant there fails here, on the
CPU, before any GPU run.  Each code u at each of the 8 positions of a dword
must decode to an exact bf16 value, and the four pair products plus the
correction must equal sum_e (u_e - 8) x_e exactly (fp64 arithmetic on bf16
inputs is exact here).  The batched router's three bf16 terms of each fp32
router weight must sum to it exactly, and their products with bf16
activations must be exact in fp32."""
import os
import re

import numpy as np

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "sparse_moe_decode_gemv_amd", "csrc", "device_common.h")


def dot2_terms(body, fn):
    """(shift, mask, magic, pair) of each `fn((word & mask) | magic, s.pN, acc)`
    term of a dot helper: the constants are named through vgpr_const(...),
    the word is w, w >> n, or a name bound to w >> n."""
    names = {m.group(1): int(m.group(2), 16) for m in re.finditer(r"(\w+) = vgpr_const\((0x[0-9A-Fa-f]+)u\)", body)}
    shifted = {m.group(1): int(m.group(2)) for m in re.finditer(r"(\w+) = w >> (\d+);", body)}
    out = []
    for m in re.finditer(fn + r"\(\(+(\w+)(?: >> (\d+)\))? ?& (\w+)\) \| (\w+), s\.p(\d)", body):
        word, sh, mask, magic, pair = m.groups()
        shift = shifted[word] if word in shifted else (int(sh) if sh else 0)
        assert word in shifted or word == "w", word
        out.append((shift, names[mask], names[magic], int(pair)))
    return out


def kernel_constants():
    src = open(HDR).read()
    body = src[src.index("float dot8("):]
    body = body[:body.index("return acc;")]
    pairs = dot2_terms(body, "dot2_bf16")
    consts = []
    for fn, var in (("make_slice(const float v[8])", "v"), ("make_slice_bf16(uint4 q)", "x")):
        mk = src[src.index(fn):]
        mk = mk[:mk.index("return s;")]
        found = re.findall(r"s\.p(\d) = pack_bf16\(\w+(?:\[\d\])? \* ([0-9.]+)f, \w+(?:\[\d\])? \* ([0-9.]+)f\)", mk)
        assert all(a == b for _, a, b in found), f"{fn}: the two halves of a pair are scaled differently"
        scale = {int(p): float(a) for p, a, _ in found}
        if var == "v":
            cm = re.search(r"s\.corr = -([0-9.]+)f \* \(\(v\[0\] \+ v\[4\]\) \+ \(v\[2\] \+ v\[6\]\)\) - "
                           r"([0-9.]+)f \* \(\(v\[1\] \+ v\[5\]\) \+ \(v\[3\] \+ v\[7\]\)\)", mk)
        else:
            cm = re.search(r"s\.corr = -([0-9.]+)f \* \(\(x0 \+ x4\) \+ \(x2 \+ x6\)\) - "
                           r"([0-9.]+)f \* \(\(x1 \+ x5\) \+ \(x3 \+ x7\)\)", mk)
        assert cm and sorted(scale) == [1, 3], f"{fn} no longer matches the expected form"
        consts.append((scale, float(cm.group(1)), float(cm.group(2))))
    assert len(pairs) == 4, "dot8 no longer matches the expected form"
    assert consts[0] == consts[1], "the two slice builders disagree"
    scale, c_even, c_odd = consts[0]
    return pairs, scale, c_even, c_odd


def bf16_value(bits16):
    return (np.asarray(bits16, np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_pairs(w, pairs):
    """For dwords w: the (low, high) bf16 values each pair instruction sees."""
    out = {}
    for shift, mask, magic, p in pairs:
        v = ((w >> np.uint32(shift)) & np.uint32(mask)) | np.uint32(magic)
        out[p] = (bf16_value(v & 0xFFFF), bf16_value(v >> 16))
    return out


# which element e each pair register carries in its (low, high) half, as the
# activation slices are built: p0=(x0,x4), p1=(x1,x5), p2=(x2,x6), p3=(x3,x7)
ELEMS = {0: (0, 4), 1: (1, 5), 2: (2, 6), 3: (3, 7)}


def test_every_code_at_every_position_decodes_exactly():
    pairs, scale, _, _ = kernel_constants()
    for e in range(8):
        u = np.zeros((16, 8), np.uint32)
        u[:, e] = np.arange(16)
        w = (u << (4 * np.arange(8, dtype=np.uint32))).sum(axis=1).astype(np.uint32)
        dec = decode_pairs(w, pairs)
        p = [q for q, (a, b) in ELEMS.items() if e in (a, b)][0]
        half = 0 if ELEMS[p][0] == e else 1
        vals = dec[p][half]
        # even positions: 128 + u (pair scale 1); odd: 128 + 8u (activation scaled by 1/8)
        f = scale.get(p, 1.0)
        np.testing.assert_array_equal(vals, 128 + np.arange(16) / f)


def test_identity_on_random_codes_and_activations():
    pairs, scale, c_even, c_odd = kernel_constants()
    rng = np.random.default_rng(5)
    n = 20000
    u = rng.integers(0, 16, size=(n, 8)).astype(np.uint32)
    w = (u << (4 * np.arange(8, dtype=np.uint32))).sum(axis=1).astype(np.uint32)
    x = bf16_value(rng.integers(0, 1 << 16, size=(n, 8)) & 0xBFFF)  # finite bf16, |x| < 2
    x[np.abs(x) < 1e-30] = 0.0
    dec = decode_pairs(w, pairs)
    acc = -c_even * (x[:, 0] + x[:, 4] + x[:, 2] + x[:, 6]) - c_odd * (x[:, 1] + x[:, 5] + x[:, 3] + x[:, 7])
    for p, (a, b) in ELEMS.items():
        f = scale.get(p, 1.0)
        acc = acc + dec[p][0] * (x[:, a] * f) + dec[p][1] * (x[:, b] * f)
    want = ((u.astype(np.int64) - 8) * x).sum(axis=1)
    np.testing.assert_allclose(acc, want, rtol=0, atol=1e-9 * np.abs(x).sum(axis=1).max())


# ---------------------------------------------------------------- fp16 variant


def fp16_constants():
    src = open(HDR).read()
    body = src[src.index("float dot8_f16("):]
    body = body[:body.index("return acc;")]
    pairs = dot2_terms(body, "dot2_f16")
    mk = src[src.index("make_slice_f16(const float v[8])"):]
    mk = mk[:mk.index("return s;")]
    found = re.findall(r"s\.p(\d) = pack_f16\(v\[\d\] \* ([0-9.]+)f, v\[\d\] \* ([0-9.]+)f\)", mk)
    assert all(a == b for _, a, b in found)
    scale = {int(p): float(a) for p, a, _ in found}
    cf = src[src.index("float slice_f16_corr("):]
    cf = cf[:cf.index("}")]
    assert "slice_f16_corr(s.p0, s.p1, s.p2, s.p3)" in mk
    cm = re.search(r"return -([0-9.]+)f \* e - ([0-9.]+)f \* o;", cf)
    assert len(pairs) == 4 and cm and sorted(scale) == [1, 3], "fp16 helpers no longer match the expected form"
    return pairs, scale, float(cm.group(1)), float(cm.group(2))


def f16_value(bits16):
    return np.asarray(bits16, np.uint16).view(np.float16).astype(np.float64)


def test_fp16_every_code_at_every_position_decodes_exactly():
    pairs, scale, _, _ = fp16_constants()
    for e in range(8):
        u = np.zeros((16, 8), np.uint32)
        u[:, e] = np.arange(16)
        w = (u << (4 * np.arange(8, dtype=np.uint32))).sum(axis=1).astype(np.uint32)
        p = [q for q, (a, b) in ELEMS.items() if e in (a, b)][0]
        shift, mask, magic, _ = [t for t in pairs if t[3] == p][0]
        v = ((w >> np.uint32(shift)) & np.uint32(mask)) | np.uint32(magic)
        half = v & 0xFFFF if ELEMS[p][0] == e else v >> 16
        np.testing.assert_array_equal(f16_value(half), 1024 + np.arange(16) / scale.get(p, 1.0))


def test_fp16_identity_on_random_codes_and_activations():
    pairs, scale, c_even, c_odd = fp16_constants()
    rng = np.random.default_rng(6)
    n = 20000
    u = rng.integers(0, 16, size=(n, 8)).astype(np.uint32)
    w = (u << (4 * np.arange(8, dtype=np.uint32))).sum(axis=1).astype(np.uint32)
    h = rng.standard_normal((n, 8))
    # activations as the kernel rounds them: fp16 of h (even) and of h*scale (odd)
    stored = np.empty_like(h)
    for p, (a, b) in ELEMS.items():
        f = scale.get(p, 1.0)
        stored[:, a] = (h[:, a] * f).astype(np.float16).astype(np.float64)
        stored[:, b] = (h[:, b] * f).astype(np.float16).astype(np.float64)
    even = stored[:, [0, 2, 4, 6]].sum(axis=1)
    odd = stored[:, [1, 3, 5, 7]].sum(axis=1)
    acc = -c_even * even - c_odd * odd
    for shift, mask, magic, p in pairs:
        v = ((w >> np.uint32(shift)) & np.uint32(mask)) | np.uint32(magic)
        a, b = ELEMS[p]
        acc = acc + f16_value(v & 0xFFFF) * stored[:, a] + f16_value(v >> 16) * stored[:, b]
    h_eff = stored.copy()
    for p, (a, b) in ELEMS.items():
        h_eff[:, a] /= scale.get(p, 1.0)
        h_eff[:, b] /= scale.get(p, 1.0)
    want = ((u.astype(np.int64) - 8) * h_eff).sum(axis=1)
    np.testing.assert_allclose(acc, want, rtol=0, atol=1e-9 * np.abs(h_eff).sum(axis=1).max())
    # and the fp16 rounding of h stays within 2^-11 relative of the fp32 value
    assert np.all(np.abs(h_eff - h) <= np.abs(h) * 2.0 ** -11 + 2.0 ** -24 * 16)


def _bf16_rne(a):
    """fp32 -> bf16 (as fp32 values), round to nearest even, as v_cvt_pk_bf16_f32 (finite inputs)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def _router_terms(w):
    """The batched router's three bf16 terms of an fp32 weight, each from what the
    previous ones left, every step in fp32 as in k_router_terms."""
    w = np.asarray(w, dtype=np.float32)
    h = _bf16_rne(w)
    r1 = (w - h).astype(np.float32)
    m = _bf16_rne(r1)
    r2 = (r1 - m).astype(np.float32)
    lo = _bf16_rne(r2)
    return h, m, lo, r2


def test_router_terms_sum_exactly_to_the_weight():
    """h + m + l == w exactly (so the three bf16 MFMAs see every router weight
    whole) over router-like N(0, 0.02) weights, a wide exponent range, and
    weights at bf16 rounding ties; and each term is a bf16 value."""
    rng = np.random.default_rng(7)
    w = np.concatenate([
        rng.normal(0, 0.02, 200000),
        rng.choice([-1.0, 1.0], 50000) * rng.uniform(1, 2, 50000) * 2.0 ** rng.integers(-100, 100, 50000),
        # ties: a bf16 value plus exactly half of its last place (and neighbours)
        (_bf16_rne(rng.normal(0, 1, 20000).astype(np.float32)).astype(np.float64)
         * (1 + 2.0 ** -8 * np.array([1.0, 1 + 2.0 ** -15, 1 - 2.0 ** -15]).repeat(20000)[:20000])),
    ]).astype(np.float32)
    h, m, lo, r2 = _router_terms(w)
    for t in (h, m, lo):
        assert np.all((t.view(np.uint32) & 0xFFFF) == 0)
    assert np.array_equal(lo, r2), "the third term must take the remainder whole"
    assert np.array_equal(h.astype(np.float64) + m.astype(np.float64) + lo.astype(np.float64), w.astype(np.float64))
    # below 2^-100 the last term can fall under bf16's normal range: an
    # absolute error below 2^-133, far under any logit's rounding
    tiny = (rng.uniform(1, 2, 10000) * 2.0 ** rng.integers(-126, -100, 10000)).astype(np.float32)
    h, m, lo, _ = _router_terms(tiny)
    err = np.abs(h.astype(np.float64) + m + lo - tiny.astype(np.float64))
    assert err.max() < 2.0 ** -133


def test_router_term_products_are_exact_in_fp32():
    """x (bf16) times a bf16 term has at most 16 significant bits: exact in fp32,
    so the MFMA's only rounding is its fp32 accumulation."""
    rng = np.random.default_rng(8)
    x = _bf16_rne(rng.normal(0, 1, 100000).astype(np.float32))
    h, m, lo, _ = _router_terms(rng.normal(0, 0.02, 100000).astype(np.float32))
    for t in (h, m, lo):
        p64 = x.astype(np.float64) * t.astype(np.float64)
        assert np.array_equal(p64.astype(np.float32).astype(np.float64), p64)
