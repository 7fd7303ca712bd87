"""Pins of the oracle's number formats: textbook bit patterns, an exhaustive
cross-check of the binary16 decoder, the stored int4 layout worked by hand,
and the quantizer's exact round trip and error bound."""
import numpy as np
import pytest

from conftest import golden_lines
from oracle import formats as F


def test_bf16_textbook_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x4049, 0x0001, 0x7F7F], np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 3.140625, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127]
    np.testing.assert_array_equal(F.bf16_to_f64(bits), want)


def test_f16_textbook_patterns():
    bits = np.array([0x3C00, 0x0001, 0x7BFF, 0x0400, 0x3555, 0xC000, 0x03FF, 0x2E66], np.uint16)
    want = [1.0, 2.0 ** -24, 65504.0, 2.0 ** -14, 0.333251953125, -2.0, 1023 * 2.0 ** -24, 0.0999755859375]
    np.testing.assert_array_equal(F.f16_to_f64(bits), want)


def test_f16_decoder_matches_numpy_on_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    finite = (bits & 0x7C00) != 0x7C00
    ours = F.f16_to_f64(bits[finite])
    ref = bits[finite].view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(ours, ref)


def test_f16_encoder_round_trips_every_finite_value():
    bits = np.arange(65536, dtype=np.uint16)
    bits = bits[(bits & 0x7C00) != 0x7C00]
    back = F.f64_to_f16_bits(F.f16_to_f64(bits))
    # -0.0 and +0.0 keep their sign bit
    np.testing.assert_array_equal(back, bits)


def test_f16_encoder_ties_to_even():
    one_ulp = 2.0 ** -10
    assert F.f64_to_f16_bits(1.0 + one_ulp / 2) == 0x3C00          # tie -> even (1.0)
    assert F.f64_to_f16_bits(1.0 + 3 * one_ulp / 2) == 0x3C02      # tie -> even (1 + 2 ulp)
    assert F.f64_to_f16_bits(2.0 ** -25) == 0x0000                 # half the smallest subnormal -> 0
    assert F.f64_to_f16_bits(3 * 2.0 ** -25) == 0x0002


def test_bf16_encoder_rounding():
    assert F.f64_to_bf16_bits(1.0) == 0x3F80
    assert F.f64_to_bf16_bits(1.0 + 2.0 ** -8) == 0x3F80           # tie -> even
    assert F.f64_to_bf16_bits(1.0 + 3 * 2.0 ** -8) == 0x3F82       # tie -> even
    assert F.f64_to_bf16_bits(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert F.f64_to_bf16_bits(-3.140625) == 0xC049
    x = np.random.default_rng(0).standard_normal(10000)
    b = F.f64_to_bf16_bits(x)
    err = np.abs(F.bf16_to_f64(b) - x)
    assert np.all(err <= np.abs(x) * 2.0 ** -8 * (1 + 1e-12))


@pytest.mark.parametrize("pattern", ["A", "B"])
def test_int4_layout_hand_worked(pattern):
    rows = {ln[0]: bytes(int(h, 16) for h in ln[1:]) for ln in golden_lines("int4_layout_k128.txt")}
    k = np.arange(128)
    u = (k // 8) % 16 if pattern == "A" else k % 8 + 8 * (k // 64)
    packed = F.pack_codes(u[None, :])[0]
    assert packed.tobytes() == rows[pattern]
    np.testing.assert_array_equal(F.unpack_codes(np.frombuffer(rows[pattern], np.uint8)[None], 128)[0], u)


def test_int4_positions_are_a_bijection():
    for K in (128, 256, 2048):
        byte, shift = F.int4_positions(K)
        slots = byte * 2 + shift // 4
        assert sorted(slots.tolist()) == list(range(K))


def test_quantize_hand_worked_group():
    lines = {ln[0]: ln[1:] for ln in golden_lines("quantize_group.txt")}
    w = np.array([float(v) for v in lines["w"]], np.float32)
    u, s = F.quantize(w[None, :])
    assert int(s[0, 0]) == int(lines["scale_bits"][0], 16)
    np.testing.assert_array_equal(u[0], [int(v) for v in lines["u"]])


def test_quantize_round_trip_exact():
    """quantize(dequant(q, s)) == (q, s) when max|q| = 7 and s is a positive
    normal binary16: q*s is exact, a = 7s, a/7 = s, so s and q come back."""
    rng = np.random.default_rng(1)
    R, K = 64, 256
    q = rng.integers(-7, 8, size=(R, K))
    q[:, ::32] = np.where(rng.random((R, K // 32)) < 0.5, 7, -7)  # every group reaches |q| = 7
    sbits = rng.integers(0x0400, 0x7800, size=(R, K // 32)).astype(np.uint16)  # normal, below 7*s overflow
    w = (q * np.repeat(F.f16_to_f64(sbits), 32, axis=1)).astype(np.float32)
    assert np.all(w.astype(np.float64) == q * np.repeat(F.f16_to_f64(sbits), 32, axis=1))
    u2, s2 = F.quantize(w)
    np.testing.assert_array_equal(s2, sbits)
    np.testing.assert_array_equal(u2 - 8, q)
    # and the packed form decodes back to the same weights
    np.testing.assert_array_equal(F.dequant(F.pack_codes(u2), s2, K), w.astype(np.float64))


def test_quantize_error_bound():
    """|w - deq(quant(w))| <= s/2 per element (s the group's stored scale),
    and the scale is within a binary16 rounding of max|w|/7."""
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((128, 512)) * 0.02).astype(np.float32)
    u, s = F.quantize(w)
    deq = F.dequant(F.pack_codes(u), s, 512)
    sv = np.repeat(F.f16_to_f64(s), 32, axis=1)
    assert np.all(np.abs(w - deq) <= sv / 2 * (1 + 1e-12))
    a = np.abs(w.reshape(128, 16, 32)).max(-1).astype(np.float64)
    assert np.all(np.abs(F.f16_to_f64(s) - a / 7) <= a / 7 * 2.0 ** -11)


def test_quantize_zero_group():
    u, s = F.quantize(np.zeros((2, 128), np.float32))
    assert np.all(s == 0) and np.all(u == 8)


# ------------------------------------------------------------------ MXFP4


def test_fp4_e2m1_every_code_against_the_spec_table():
    """All 16 codes against the E2M1 table written out from the MX
    specification (tests/golden/fp4_e2m1.txt), signed zero included."""
    rows = golden_lines("fp4_e2m1.txt")
    codes = np.array([int(r[0]) for r in rows])
    want = np.array([float(r[1]) for r in rows])
    got = F.fp4_e2m1_to_f64(codes)
    assert len(codes) == 16 and np.array_equal(np.sort(codes), np.arange(16))
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))


def test_e8m0_scales_match_fp32_exponent_patterns():
    """2^(b-127) for every byte: b = 1..254 is the fp32 pattern b << 23, b = 0
    the subnormal 0x00400000 (2^-127), b = 255 NaN."""
    b = np.arange(256)
    got = F.e8m0_to_f64(b)
    want = np.empty(256)
    want[1:255] = (b[1:255].astype(np.uint32) << 23).view(np.float32)
    want[0] = np.array([0x00400000], np.uint32).view(np.float32)[0]
    assert np.array_equal(got[:255], want[:255]) and np.isnan(got[255])


def test_mxfp4_dequant_hand_worked_row():
    """One 128-element row: code 7 (6.0) at element 37 with scale byte 125
    (1/4) in its block 1, code 9 (-0.5) at element 100 with scale byte 130 (8)
    in block 3: w[37] = 1.5, w[100] = -4, every other element 0."""
    u = np.zeros((1, 128), np.int64)
    u[0, 37], u[0, 100] = 7, 9
    s = np.array([[127, 125, 127, 130]], np.uint8)
    w = F.dequant_mxfp4(F.pack_codes(u), s, 128)[0]
    want = np.zeros(128)
    want[37], want[100] = 1.5, -4.0
    assert np.array_equal(w, want)


def test_mxfp4_quantize_matches_brute_force():
    """Shared exponent floor(log2 amax) - 2 (computed here with frexp) and
    every element the nearest of the 16 codes' values at that scale, ties
    to the even code, over random blocks of many magnitudes."""
    rng = np.random.default_rng(11)
    w = (rng.normal(0, 1, (64, 128)) * 2.0 ** rng.integers(-20, 10, (64, 1))).astype(np.float32)
    w[3, :32] = 0.0  # one all-zero block
    codes, sb = F.quantize_mxfp4(w)
    vals = F.fp4_e2m1_to_f64(np.arange(16))
    for r in range(w.shape[0]):
        for g in range(4):
            blk = w[r, 32 * g:32 * g + 32].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                assert sb[r, g] == 127 and np.all(codes[r, 32 * g:32 * g + 32] == 0)
                continue
            _, e = np.frexp(amax)          # amax = m 2^e, 0.5 <= m < 1: floor(log2 amax) = e - 1
            assert sb[r, g] == e - 1 - 2 + 127
            scale = 2.0 ** (int(sb[r, g]) - 127)
            for i, x in enumerate(blk):
                d = np.abs(x - vals * scale)
                d[8] = np.inf  # -0 is never chosen
                best = np.flatnonzero(d == d.min())
                pick = best[best % 2 == 0][0] if np.any(best % 2 == 0) else best[0]
                assert F.fp4_e2m1_to_f64(codes[r, 32 * g + i]) == vals[pick], (r, g, i, x)


def test_mxfp4_representable_values_round_trip():
    """Weights that are MXFP4 values already come back unchanged (possibly
    with another code/scale pair of equal value)."""
    rng = np.random.default_rng(12)
    u = rng.integers(0, 16, (32, 256))
    s = rng.integers(100, 140, (32, 8)).astype(np.uint8)
    w = F.dequant_mxfp4(F.pack_codes(u), s, 256)
    c2, s2 = F.quantize_mxfp4(w.astype(np.float32))
    assert np.array_equal(F.dequant_mxfp4(F.pack_codes(c2), s2, 256), w)


def test_mxfp4_quantize_saturates_at_six():
    """amax / 2^X lies in [4, 8): a block whose largest element is 7.9 * 2^X
    stores it as 6 * 2^X (the largest E2M1 magnitude)."""
    w = np.zeros((1, 32), np.float32)
    w[0, 0], w[0, 1] = 7.9, -7.9
    c, s = F.quantize_mxfp4(w)
    assert s[0, 0] == 127 and c[0, 0] == 7 and c[0, 1] == 15


# ------------------------------------------------------------------ NVFP4


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    """All 256 E4M3 bytes against torch's float8_e4m3fn (the OCP E4M3FN
    type): equal values and signs, NaN exactly at S.1111.111."""
    import torch
    b = np.arange(256)
    got = F.e4m3_to_f64(b)
    want = torch.from_numpy(b.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    nan = (b & 0x7F) == 0x7F
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(np.isnan(want), nan)
    assert np.array_equal(got[~nan], want[~nan]) and np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_e4m3_encoder_matches_torch_rounding():
    """The quantizer's E4M3 rounding (nearest, ties to even) against torch's
    float -> float8_e4m3fn cast on values in [0, 448], ties included."""
    import torch
    rng = np.random.default_rng(13)
    vals = F.e4m3_to_f64(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([rng.uniform(0, 448, 4000), rng.uniform(0, 2 ** -5, 2000), mids, vals])
    got = F.e4m3_to_f64(F.f64_to_e4m3(x))
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(got, want)


def test_nvfp4_dequant_hand_worked_row():
    """One 128-element row: code 5 (3.0) at element 20 in block 1 with scale
    byte 0x40 (E4M3 2.0), code 14 (-4.0) at element 71 in block 4 with scale
    byte 0x31 (1.125 * 2^-1 = 0.5625), tensor scale 0.25:
    w[20] = 3 * 2 * 0.25 = 1.5, w[71] = -4 * 0.5625 * 0.25 = -0.5625."""
    u = np.zeros((1, 128), np.int64)
    u[0, 20], u[0, 71] = 5, 14
    s = np.zeros((1, 8), np.uint8)
    s[0, 1], s[0, 4] = 0x40, 0x31
    w = F.dequant_nvfp4(F.pack_codes(u), s, np.float32(0.25), 128)[0]
    want = np.zeros(128)
    want[20], want[71] = 1.5, -0.5625
    assert np.array_equal(w, want)


def test_nvfp4_quantize_matches_brute_force():
    """Tensor scale amax / (6 * 448) in fp32; every block's scale the E4M3
    value nearest to amax(block) / 6 / t; every element the nearest E2M1
    value at that scale (ties to the even code)."""
    rng = np.random.default_rng(14)
    w = (rng.normal(0, 1, (16, 128)) * 2.0 ** rng.integers(-6, 3, (16, 8)).repeat(16, axis=1)).astype(np.float32)
    codes, sb, t = F.quantize_nvfp4(w)
    assert t == np.float32(np.abs(w.astype(np.float64)).max() / (6 * 448))
    e4 = F.e4m3_to_f64(np.arange(0x7F))
    vals = F.fp4_e2m1_to_f64(np.arange(16))
    for r in range(16):
        for g in range(8):
            blk = w[r, 16 * g:16 * g + 16].astype(np.float64)
            target = np.abs(blk).max() / 6.0 / np.float64(t)
            dd = np.abs(e4 - target)
            best = np.flatnonzero(dd == dd.min())
            pick = best[best % 2 == 0][0] if np.any(best % 2 == 0) else best[0]
            assert sb[r, g] == pick, (r, g)
            scale = e4[pick] * np.float64(t)
            for i, x in enumerate(blk):
                d = np.abs(x - vals * scale)
                d[8] = np.inf
                b2 = np.flatnonzero(d == d.min())
                p2 = b2[b2 % 2 == 0][0] if np.any(b2 % 2 == 0) else b2[0]
                assert F.fp4_e2m1_to_f64(codes[r, 16 * g + i]) == vals[p2], (r, g, i)
