"""Number formats of the decode path, decoded by their definitions (fp64).

TEST INFRASTRUCTURE ONLY: part of the plain CPU oracle.  Nothing in the
product path may import this package.

The pages list 4-bit integer builds among the releases and say the output layer
is quantized to 4 bits ("Flint 40B: Best Mid Sized LLM", transcript 05:39 and
07:15; "Recursive Releases Flint...", section "Built by an Automated Research
System").  They give no group size, scale type or nibble order, so the stored
format is a stated choice:

* symmetric int4 codes, one fp16 scale per group of 32 consecutive elements
  along K; weight = (u - 8) * scale with stored code u in 0..15;
* rows of K elements (K a multiple of 128) take K/2 bytes; element k of a row
  sits in byte 64*t + 16*q + 4*j + e//2 with t = k//128, j = (k%128)//32,
  q = (k%32)//8, e = k%8, low nibble for even e, high nibble for odd e;
* scales are IEEE binary16 bit patterns, row-major [rows][K/32].

Quantizer (offline, produces stored weights): per group a = max|w|,
s = fp16_RNE(a/7) with a/7 in fp64; s == 0 gives all codes 8, otherwise
q = clamp(round_half_even(w/s), -7, 7) and u = q + 8.

The pages name NVFP4 as the released model's 4-bit format ("Recursive
Releases Flint...", section "Quantization"; noticiai.com.br page, section "O
papel da quantização e dos kernels") without defining it.  The FP4 variant
here is MXFP4, the OCP Microscaling (MX) v1.0 format, whose block scale the
target hardware decodes natively:

* element: FP4 E2M1, 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit;
  exponent field e > 0 gives (-1)^s 2^(e-1) (1 + m/2), e = 0 gives (-1)^s m/2;
  no infinities or NaN (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6);
* scale: E8M0, an unsigned byte b standing for 2^(b-127) (b = 255 is NaN);
  one scale per 32 consecutive elements along K;
* stored: codes at the int4 nibble positions above, scale bytes [rows][K/32].

NVFP4 (the format the pages name; its public definition): the same E2M1
codes at the same positions, one FP8 E4M3 scale per 16 elements along K
(OCP E4M3FN: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
448, S.1111.111 is NaN, no infinity) and one fp32 scale per tensor (here per
expert matrix); w = e2m1(c) * e4m3(s_block) * s_tensor.  Stored: codes as
above, scale bytes [rows][K/16], tensor scales fp32 [E].  Its two-level
quantizer: s_tensor = amax(matrix) / (6 * 448); per block the E4M3 value
nearest to amax(block) / 6 / s_tensor (ties to even, at most 448); then each
element w / (e4m3(s_block) * s_tensor) to the nearest E2M1 value as for
MXFP4; a zero block (or matrix) gets scale 0 and codes 0.

MXFP4 quantizer (the MX specification's conversion): per block a = max|w|;
a == 0 gives scale byte 127 and all codes 0; otherwise the shared exponent is
X = floor(log2 a) - 2 (2 = the largest E2M1 exponent), the scale byte X + 127
(clamped to 0..254), and every element w / 2^X goes to the nearest E2M1
value, ties to the even mantissa, magnitudes above 6 to 6.
"""
from __future__ import annotations

import numpy as np


# ------------------------------------------------------------------ floats


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> fp64.  A bf16 value is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_to_f64(bits) -> np.ndarray:
    """IEEE-754 binary16 bit patterns -> fp64 from the definition
    (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    ex = (b >> 10) & 0x1F
    fr = (b & 0x3FF).astype(np.float64)
    normal = sign * (1.0 + fr / 1024.0) * np.exp2(ex.astype(np.float64) - 15.0)
    subnormal = sign * (fr / 1024.0) * 2.0 ** -14
    special = np.where(fr == 0, sign * np.inf, np.nan)
    return np.where(ex == 0, subnormal, np.where(ex == 31, special, normal))


def f64_to_f16_bits(x) -> np.ndarray:
    """fp64 -> binary16 bits, round to nearest even (numpy's conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f64_to_bf16_bits(x) -> np.ndarray:
    """fp64 -> bfloat16 bits, round to nearest even on the 8-bit significand.
    Finite inputs within bf16's normal range (all the path produces)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0)                  # 8 significant bits, ties to even
    y = np.ldexp(r / 256.0, e)              # exact
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f64_to_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# ------------------------------------------------------------------ int4


def int4_positions(K: int):
    """(byte index within a row, bit shift) of each element k = 0..K-1."""
    assert K % 128 == 0
    k = np.arange(K)
    t, j, q, e = k // 128, (k % 128) // 32, (k % 32) // 8, k % 8
    byte = 64 * t + 16 * q + 4 * j + e // 2
    shift = 4 * (e % 2)
    return byte, shift


def unpack_codes(qbytes: np.ndarray, K: int) -> np.ndarray:
    """Stored bytes [..., K/2] -> codes u [..., K] in 0..15 (uint8)."""
    byte, shift = int4_positions(K)
    b = np.asarray(qbytes, dtype=np.uint8)[..., byte]
    return (b >> shift.astype(np.uint8)) & np.uint8(0xF)


def pack_codes(u: np.ndarray) -> np.ndarray:
    """Codes u [..., K] in 0..15 -> stored bytes [..., K/2]."""
    u = np.asarray(u, dtype=np.int64)
    K = u.shape[-1]
    byte, shift = int4_positions(K)
    out = np.zeros(u.shape[:-1] + (K // 2,), dtype=np.int64)
    for k in range(K):
        out[..., byte[k]] |= u[..., k] << shift[k]
    return out.astype(np.uint8)


def dequant(qbytes: np.ndarray, sbits: np.ndarray, K: int) -> np.ndarray:
    """Stored int4 matrix -> fp64 weights [..., K]: w = (u - 8) * s[k // 32]."""
    q = unpack_codes(qbytes, K).astype(np.int8) - np.int8(8)
    s = f16_to_f64(sbits)
    return (q.reshape(q.shape[:-1] + (K // 32, 32)) * s[..., None]).reshape(q.shape)


def quantize(w: np.ndarray):
    """fp32 weights [..., K] -> (codes u [..., K], scale bits [..., K/32])."""
    w = np.asarray(w, dtype=np.float32)
    K = w.shape[-1]
    g = w.reshape(w.shape[:-1] + (K // 32, 32)).astype(np.float64)
    a = np.abs(g).max(axis=-1)
    sbits = f64_to_f16_bits(a / 7.0)
    s = f16_to_f64(sbits)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(np.rint(g / s), -7, 7)
    q = np.where(s == 0.0, 0.0, q)
    u = (q + 8).astype(np.int64).reshape(w.shape)
    return u, sbits


# ------------------------------------------------------------------ MXFP4


def fp4_e2m1_to_f64(codes) -> np.ndarray:
    """FP4 E2M1 codes (0..15) -> fp64 from the bit fields."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    normal = np.exp2(e.astype(np.float64) - 1.0) * (1.0 + m / 2.0)
    return sign * np.where(e == 0, m / 2.0, normal)


def e8m0_to_f64(b) -> np.ndarray:
    """E8M0 scale bytes -> fp64: 2^(b - 127), NaN for b = 255."""
    b = np.asarray(b, dtype=np.int64)
    return np.where(b == 255, np.nan, np.exp2(b.astype(np.float64) - 127.0))


def dequant_mxfp4(qbytes: np.ndarray, sbytes: np.ndarray, K: int) -> np.ndarray:
    """Stored MXFP4 matrix -> fp64 weights [..., K]: w = e2m1(c) * 2^(b[k // 32] - 127)."""
    v = fp4_e2m1_to_f64(unpack_codes(qbytes, K))
    s = e8m0_to_f64(sbytes)
    return (v.reshape(v.shape[:-1] + (K // 32, 32)) * s[..., None]).reshape(v.shape)


E2M1_MAGNITUDES = fp4_e2m1_to_f64(np.arange(8))


def quantize_mxfp4(w: np.ndarray):
    """fp32 weights [..., K] -> (E2M1 codes [..., K], E8M0 scale bytes [..., K/32])."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    K = w.shape[-1]
    g = w.reshape(w.shape[:-1] + (K // 32, 32))
    a = np.abs(g).max(axis=-1)
    with np.errstate(divide="ignore"):
        X = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))) - 2, 0)
    b = np.clip(X + 127, 0, 254).astype(np.int64)
    v = np.abs(g) / np.exp2(b - 127.0)[..., None]
    # nearest magnitude; on a tie the even code (even mantissa) wins
    dist = np.abs(v[..., None] - E2M1_MAGNITUDES)
    best = dist.min(axis=-1, keepdims=True)
    cand = np.where(dist == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    code = np.where(even < 99, even, cand.min(axis=-1))
    code = np.where((g < 0) & (code > 0), code | 8, code)
    code = np.where(a[..., None] > 0, code, 0)
    b = np.where(a > 0, b, 127)
    return code.reshape(w.shape).astype(np.int64), b.astype(np.uint8)


# ------------------------------------------------------------------ NVFP4


def e4m3_to_f64(b) -> np.ndarray:
    """FP8 E4M3 (OCP E4M3FN) bytes -> fp64 from the bit fields; S.1111.111 is NaN."""
    b = np.asarray(b, dtype=np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((b & 0x7F) == 0x7F, np.nan, sign * val)


E4M3_POSITIVE = e4m3_to_f64(np.arange(0x7F))  # codes 0x00..0x7E, ascending


def f64_to_e4m3(x) -> np.ndarray:
    """Non-negative fp64 -> nearest E4M3 byte (ties to the even code), saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    dist = np.abs(x[..., None] - E4M3_POSITIVE)
    best = dist.min(axis=-1, keepdims=True)
    cand = np.where(dist == best, np.arange(0x7F), 999)
    even = np.where(cand % 2 == 0, cand, 999).min(axis=-1)
    return np.where(even < 999, even, cand.min(axis=-1)).astype(np.uint8)


def dequant_nvfp4(qbytes: np.ndarray, sbytes: np.ndarray, tscale, K: int) -> np.ndarray:
    """Stored NVFP4 matrix -> fp64 weights [..., K]: e2m1(c) * e4m3(s[k // 16]) * tscale."""
    v = fp4_e2m1_to_f64(unpack_codes(qbytes, K))
    s = e4m3_to_f64(sbytes)
    w = (v.reshape(v.shape[:-1] + (K // 16, 16)) * s[..., None]).reshape(v.shape)
    t = np.asarray(tscale, dtype=np.float32).astype(np.float64)
    return w * t.reshape(t.shape + (1,) * (w.ndim - t.ndim))


def nearest_e2m1_codes(v: np.ndarray) -> np.ndarray:
    """Signed values -> nearest E2M1 code (ties to the even code, |v| > 6 to 6, zero -> code 0)."""
    a = np.abs(v)
    dist = np.abs(a[..., None] - E2M1_MAGNITUDES)
    best = dist.min(axis=-1, keepdims=True)
    cand = np.where(dist == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    code = np.where(even < 99, even, cand.min(axis=-1))
    return np.where((v < 0) & (code > 0), code | 8, code).astype(np.int64)


def quantize_nvfp4(w: np.ndarray):
    """fp32 matrix [rows][K] -> (E2M1 codes [rows][K], E4M3 scale bytes [rows][K/16], fp32 tensor scale)."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    rows, K = w.shape
    t = np.float32(np.abs(w).max() / (6.0 * 448.0))
    if t == 0:
        return np.zeros((rows, K), np.int64), np.zeros((rows, K // 16), np.uint8), np.float32(0.0)
    g = w.reshape(rows, K // 16, 16)
    sb = f64_to_e4m3(np.abs(g).max(axis=-1) / 6.0 / np.float64(t))
    s = e4m3_to_f64(sb) * np.float64(t)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s[..., None] > 0, g / s[..., None], 0.0)
    return nearest_e2m1_codes(v).reshape(rows, K), sb, t
