// device_common.h -- device helpers shared by the decode kernels (gfx950, wave64).
//
// int4 x bf16 dot products without integer->float conversions.  A stored
// 16-byte piece of a row holds, for each of 4 consecutive groups j, one
// dword w of 8 codes u_e (e = 0..7, byte e/2, low nibble for even e, so u_e
// sits in bits 4e..4e+3).  bf16 128.0 is 0x4300: exponent 2^7 and 7
// fraction bits (bits 0..6) worth 1 each.  A nibble placed in bits 0..3 of
// the fraction gives 128+u; placed in bits 3..6 it gives 128+8u.  So
//   (w        & 0x000F000F) | 0x43004300 -> bf16 pair (128+u0,  128+u4)
//   ((w >> 1) & 0x00780078) | 0x43004300 -> bf16 pair (128+8u1, 128+8u5)
//   ((w >> 8) & 0x000F000F) | 0x43004300 -> bf16 pair (128+u2,  128+u6)
//   ((w >> 9) & 0x00780078) | 0x43004300 -> bf16 pair (128+8u3, 128+8u7)
// are exact, and one v_dot2_f32_bf16 multiplies each pair by the matching
// activations, taken as x for the even positions and x/8 (exact) for the odd
// ones.  Since (128+u)x = 128x + ux and (128+8u)(x/8) = 16x + ux, the dot
// products start from
//   corr = -136 * (x0 + x2 + x4 + x6) - 24 * (x1 + x3 + x5 + x7)
// so the accumulated value is sum_e (u_e - 8) x_e up to fp32 rounding; the
// group's binary16 scale multiplies it afterwards.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16(f, 0.f) & 0xFFFFu; }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// Activations of one lane for one group: the 8 elements e = 0..7 prepared as
// the four bf16 pairs (x0,x4), (x1/8,x5/8), (x2,x6), (x3/8,x7/8) and the
// offset correction.
struct Slice8 {
  uint32_t p0, p1, p2, p3;
  float corr;
};

// From 8 fp32 values that are exactly representable in bf16.
__device__ __forceinline__ Slice8 make_slice(const float v[8]) {
  Slice8 s;
  s.p0 = pack_bf16(v[0], v[4]);
  s.p1 = pack_bf16(v[1] * 0.125f, v[5] * 0.125f);
  s.p2 = pack_bf16(v[2], v[6]);
  s.p3 = pack_bf16(v[3] * 0.125f, v[7] * 0.125f);
  s.corr = -136.0f * ((v[0] + v[4]) + (v[2] + v[6])) - 24.0f * ((v[1] + v[5]) + (v[3] + v[7]));
  return s;
}

// From 8 bf16 values held as 4 dwords (dword i = elements 2i (low), 2i+1 (high)).
__device__ __forceinline__ Slice8 make_slice_bf16(uint4 q) {
  Slice8 s;
  s.p0 = (q.x & 0xFFFFu) | (q.z << 16);
  s.p2 = (q.y & 0xFFFFu) | (q.w << 16);
  const float x0 = bf16_bits_to_f32(q.x & 0xFFFFu), x1 = __uint_as_float(q.x & 0xFFFF0000u);
  const float x2 = bf16_bits_to_f32(q.y & 0xFFFFu), x3 = __uint_as_float(q.y & 0xFFFF0000u);
  const float x4 = bf16_bits_to_f32(q.z & 0xFFFFu), x5 = __uint_as_float(q.z & 0xFFFF0000u);
  const float x6 = bf16_bits_to_f32(q.w & 0xFFFFu), x7 = __uint_as_float(q.w & 0xFFFF0000u);
  s.p1 = pack_bf16(x1 * 0.125f, x5 * 0.125f);
  s.p3 = pack_bf16(x3 * 0.125f, x7 * 0.125f);
  s.corr = -136.0f * ((x0 + x4) + (x2 + x6)) - 24.0f * ((x1 + x5) + (x3 + x7));
  return s;
}

// A constant held in a VGPR the compiler cannot see through.  gfx950's
// three-operand (VOP3) encodings take no 32-bit literal, so (w & mask) |
// magic with literal constants compiles to a v_and and a v_or; with both
// constants in VGPRs it is one v_and_or_b32.  (The empty asm has no side
// effect, so repeated uses are merged and hoisted out of loops.)
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

// acc + sum_e (128+u_e or 128+8u_e) * (x_e or x_e/8); started from s.corr
// this is sum_e (u_e - 8) x_e.
__device__ __forceinline__ float dot8(uint32_t w, const Slice8& s, float acc) {
  const uint32_t lo = vgpr_const(0x000F000Fu), mid = vgpr_const(0x00780078u), mg = vgpr_const(0x43004300u);
  acc = dot2_bf16((w & lo) | mg, s.p0, acc);
  acc = dot2_bf16(((w >> 1) & mid) | mg, s.p1, acc);
  acc = dot2_bf16(((w >> 8) & lo) | mg, s.p2, acc);
  acc = dot2_bf16(((w >> 9) & mid) | mg, s.p3, acc);
  return acc;
}

// One 16-byte piece (4 groups x 8 codes) against 4 prepared slices, scaled by
// the 4 groups' binary16 scales (sc.x = groups 0,1; sc.y = groups 2,3).
__device__ __forceinline__ float dot_piece(uint4 q, const Slice8 xs[4], uint2 sc) {
  // the first product as an fma with +0 as well: one v_fma_mix_f32 (binary16
  // operand) rather than a conversion and a multiply
  float p = fmaf(dot8(q.x, xs[0], xs[0].corr), f16_bits_to_f32(sc.x & 0xFFFFu), 0.f);
  p = fmaf(dot8(q.y, xs[1], xs[1].corr), f16_bits_to_f32(sc.x >> 16), p);
  p = fmaf(dot8(q.z, xs[2], xs[2].corr), f16_bits_to_f32(sc.y & 0xFFFFu), p);
  p = fmaf(dot8(q.w, xs[3], xs[3].corr), f16_bits_to_f32(sc.y >> 16), p);
  return p;
}

// ---- fp16 variant for internally produced activations (the SwiGLU output h)
// fp16 1024.0 is 0x6400: 10 fraction bits worth 1 each, so a nibble in bits
// 0..3 gives 1024+u and in bits 4..7 gives 1024+16u -- both exact, and only
// one shift per dword is needed:
//   (w        & 0x000F000F) | 0x64006400 -> fp16 pair (1024+u0,   1024+u4)
//   (w        & 0x00F000F0) | 0x64006400 -> fp16 pair (1024+16u1, 1024+16u5)
//   ((w >> 8) & 0x000F000F) | 0x64006400 -> fp16 pair (1024+u2,   1024+u6)
//   ((w >> 8) & 0x00F000F0) | 0x64006400 -> fp16 pair (1024+16u3, 1024+16u7)
// with activations h (even positions) and h/16 (odd), rounded to fp16
// (|h| < 65504; relative error <= 2^-11).  (1024+u)h = 1024h + uh and
// (1024+16u)(h/16) = 64h + uh, so the products start from
//   corr = -1032 * (h0 + h2 + h4 + h6) - 72 * (h1 + h3 + h5 + h7)
// taken from the rounded values, which cancels the offsets exactly.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}
__device__ __forceinline__ float f16_lo(uint32_t p) { return (float)__builtin_bit_cast(f16x2_t, p).x; }
__device__ __forceinline__ float f16_hi(uint32_t p) { return (float)__builtin_bit_cast(f16x2_t, p).y; }

// The offset correction of a slice from its 4 binary16 pairs.
__device__ __forceinline__ float slice_f16_corr(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3) {
  const float e = (f16_lo(p0) + f16_hi(p0)) + (f16_lo(p2) + f16_hi(p2));
  const float o = (f16_lo(p1) + f16_hi(p1)) + (f16_lo(p3) + f16_hi(p3));
  return -1032.0f * e - 1152.0f * o;  // odd terms are stored /16: -72 * 16
}

// From 8 fp32 activations (rounded to fp16 here).
__device__ __forceinline__ Slice8 make_slice_f16(const float v[8]) {
  Slice8 s;
  s.p0 = pack_f16(v[0], v[4]);
  s.p1 = pack_f16(v[1] * 0.0625f, v[5] * 0.0625f);
  s.p2 = pack_f16(v[2], v[6]);
  s.p3 = pack_f16(v[3] * 0.0625f, v[7] * 0.0625f);
  s.corr = slice_f16_corr(s.p0, s.p1, s.p2, s.p3);
  return s;
}

// Binary16 operands built from bf16 activations carry x 2^(a + kXf16Shift),
// a from the row's largest magnitude (act_exponent: that magnitude times 2^a
// lies in [1, 2)), so the largest lies in [2^14, 2^15).
constexpr int kXf16Shift = 14;

// acc + sum_e (1024+u_e or 1024+16u_e) * (h_e or h_e/16); started from
// s.corr this is sum_e (u_e - 8) h_e.
__device__ __forceinline__ float dot8_f16(uint32_t w, const Slice8& s, float acc) {
  const uint32_t lo = vgpr_const(0x000F000Fu), hi = vgpr_const(0x00F000F0u), mg = vgpr_const(0x64006400u);
  const uint32_t w8 = w >> 8;
  acc = dot2_f16((w & lo) | mg, s.p0, acc);
  acc = dot2_f16((w & hi) | mg, s.p1, acc);
  acc = dot2_f16((w8 & lo) | mg, s.p2, acc);
  acc = dot2_f16((w8 & hi) | mg, s.p3, acc);
  return acc;
}

__device__ __forceinline__ float dot_piece_f16(uint4 q, const Slice8 xs[4], uint2 sc) {
  float p = fmaf(dot8_f16(q.x, xs[0], xs[0].corr), f16_bits_to_f32(sc.x & 0xFFFFu), 0.f);
  p = fmaf(dot8_f16(q.y, xs[1], xs[1].corr), f16_bits_to_f32(sc.x >> 16), p);
  p = fmaf(dot8_f16(q.z, xs[2], xs[2].corr), f16_bits_to_f32(sc.y & 0xFFFFu), p);
  p = fmaf(dot8_f16(q.w, xs[3], xs[3].corr), f16_bits_to_f32(sc.y >> 16), p);
  return p;
}

// ---------------------------------------------------------------- MXFP4
// FP4 E2M1 codes at the int4 nibble positions (byte b of a dword holds the
// elements 2b, low nibble, and 2b+1), one E8M0 scale byte 2^(b-127) per 32
// elements.  gfx950 turns a byte's two codes into a bf16 or fp16 pair in one
// instruction (exact: E2M1 values have two significant bits, so products
// with bf16 or fp16 activations are exact in fp32), and the block scale
// multiplies the block's fp32 sum through ldexp (exact).  Activation slices
// hold their 8 values as they are, pairs (v0,v1) .. (v6,v7).

template <int B>
__device__ __forceinline__ uint32_t fp4_pair_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B));
}
template <int B>
__device__ __forceinline__ uint32_t fp4_pair_f16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B));
}

// 8 bf16 activations as stored (4 pairs).
__device__ __forceinline__ Slice8 make_slice_raw(uint4 q) { return Slice8{q.x, q.y, q.z, q.w, 0.f}; }

// From 8 fp32 activations, rounded to fp16, in pairs.
__device__ __forceinline__ Slice8 make_slice_f16_raw(const float v[8]) {
  return Slice8{pack_f16(v[0], v[1]), pack_f16(v[2], v[3]), pack_f16(v[4], v[5]), pack_f16(v[6], v[7]), 0.f};
}

__device__ __forceinline__ float e8m0_scaled(float v, uint32_t sc, int j) {
  return ldexpf(v, (int)((sc >> (8 * j)) & 0xFFu) - 127);
}

// sum_e e2m1(c_e) x_e over one dword's 8 codes
__device__ __forceinline__ float dot8_fp4(uint32_t w, const Slice8& s) {
  float acc = dot2_bf16(fp4_pair_bf16<0>(w), s.p0, 0.f);
  acc = dot2_bf16(fp4_pair_bf16<1>(w), s.p1, acc);
  acc = dot2_bf16(fp4_pair_bf16<2>(w), s.p2, acc);
  return dot2_bf16(fp4_pair_bf16<3>(w), s.p3, acc);
}
__device__ __forceinline__ float dot8_fp4_f16(uint32_t w, const Slice8& s) {
  float acc = dot2_f16(fp4_pair_f16<0>(w), s.p0, 0.f);
  acc = dot2_f16(fp4_pair_f16<1>(w), s.p1, acc);
  acc = dot2_f16(fp4_pair_f16<2>(w), s.p2, acc);
  return dot2_f16(fp4_pair_f16<3>(w), s.p3, acc);
}

// NVFP4: an OCP E4M3 scale per 16 elements; the 4 dwords of a piece take
// the bytes 0, 2, 4, 6 of `sc` (the piece's 8 scale bytes shifted so that
// its own come first); products rounded once in fp32.  e4m3_f32 decodes
// with integer operations (used at init); the dot products use gfx950's
// fp8 conversion, which on this target decodes the OCP E4M3 format exactly,
// in one instruction with a byte select.
__device__ __forceinline__ float e4m3_f32(uint32_t b) {
  const uint32_t em = b & 0x7Fu;
  const float mag = em >= 8u ? __uint_as_float((em + (120u << 3)) << 20) : (float)em * 0.001953125f;
  return (b & 0x80u) ? -mag : mag;
}
template <int BYTE>
__device__ __forceinline__ float e4m3_byte(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, BYTE);
}
__device__ __forceinline__ float dot_piece_nv(uint4 q, const Slice8 xs[4], uint2 sc) {
  float p = dot8_fp4(q.x, xs[0]) * e4m3_byte<0>(sc.x);
  p = fmaf(dot8_fp4(q.y, xs[1]), e4m3_byte<2>(sc.x), p);
  p = fmaf(dot8_fp4(q.z, xs[2]), e4m3_byte<0>(sc.y), p);
  p = fmaf(dot8_fp4(q.w, xs[3]), e4m3_byte<2>(sc.y), p);
  return p;
}
__device__ __forceinline__ float dot_piece_nv_f16(uint4 q, const Slice8 xs[4], uint2 sc) {
  float p = dot8_fp4_f16(q.x, xs[0]) * e4m3_byte<0>(sc.x);
  p = fmaf(dot8_fp4_f16(q.y, xs[1]), e4m3_byte<2>(sc.x), p);
  p = fmaf(dot8_fp4_f16(q.z, xs[2]), e4m3_byte<0>(sc.y), p);
  p = fmaf(dot8_fp4_f16(q.w, xs[3]), e4m3_byte<2>(sc.y), p);
  return p;
}

// One 16-byte piece (dword j in scale block j of the four) against bf16
// (dot_piece_fp4) or fp16 (dot_piece_fp4_f16) slices; sc = the 4 scale bytes.
__device__ __forceinline__ float dot_piece_fp4(uint4 q, const Slice8 xs[4], uint32_t sc) {
  float p = e8m0_scaled(dot8_fp4(q.x, xs[0]), sc, 0);
  p += e8m0_scaled(dot8_fp4(q.y, xs[1]), sc, 1);
  p += e8m0_scaled(dot8_fp4(q.z, xs[2]), sc, 2);
  p += e8m0_scaled(dot8_fp4(q.w, xs[3]), sc, 3);
  return p;
}
__device__ __forceinline__ float dot_piece_fp4_f16(uint4 q, const Slice8 xs[4], uint32_t sc) {
  float p = e8m0_scaled(dot8_fp4_f16(q.x, xs[0]), sc, 0);
  p += e8m0_scaled(dot8_fp4_f16(q.y, xs[1]), sc, 1);
  p += e8m0_scaled(dot8_fp4_f16(q.z, xs[2]), sc, 2);
  p += e8m0_scaled(dot8_fp4_f16(q.w, xs[3]), sc, 3);
  return p;
}

// ---- cross-lane reductions (VALU only: DPP and gfx950 permlane swaps) ------
// Steps pair lanes within growing aligned segments: quad_perm [1,0,3,2] and
// [2,3,0,1] (segments of 2 and 4), row_half_mirror (8), row_mirror (16),
// v_permlane16_swap (32: rows 0<->1 and 2<->3) and v_permlane32_swap (64:
// the two half-waves).  After each step every lane of a segment holds the
// same value, so the mirror pairings (lane i with 7-i, 15-i) combine the two
// halves like an xor would.  No step goes through LDS or the scalar unit.
enum : int { kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140 };

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// (value of this lane, value of the lane 16 rows away) for xor-16 pairing
__device__ __forceinline__ u32x2_t swap16(uint32_t v) { return __builtin_amdgcn_permlane16_swap(v, v, false, false); }
__device__ __forceinline__ u32x2_t swap32(uint32_t v) { return __builtin_amdgcn_permlane32_swap(v, v, false, false); }

// Sum over aligned segments of SEG lanes (SEG a power of two <= 64); every
// lane of a segment receives the segment's sum.
template <int SEG>
__device__ __forceinline__ float seg_sum(float v) {
  if constexpr (SEG >= 2) v += dpp_f<kDppXor1>(v);
  if constexpr (SEG >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (SEG >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (SEG >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (SEG >= 32) {
    const u32x2_t p = swap16(__float_as_uint(v));
    v = __uint_as_float(p.x) + __uint_as_float(p.y);
  }
  if constexpr (SEG >= 64) {
    const u32x2_t p = swap32(__float_as_uint(v));
    v = __uint_as_float(p.x) + __uint_as_float(p.y);
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return seg_sum<64>(v); }

// Eight wave sums at once (reduce-scatter): lane l receives the sum over
// the wave of v[(l >> 3) & 7].  Each permlane swap exchanges two different
// values, so a halving step costs one swap and one add per pair of values:
// 18 instructions instead of the 8 x 8 of separate sums.
__device__ __forceinline__ float wave_sum8_scatter(const float v[8]) {
  const int lane = threadIdx.x & 63;
  float a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // half-waves: lanes 0-31 keep values 0-3, lanes 32-63 values 4-7
    const u32x2_t p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 4]), false, false);
    a[i] = __uint_as_float(p.x) + __uint_as_float(p.y);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // 16-lane rows: even rows keep a[0..1], odd rows a[2..3]
    const u32x2_t p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]), __float_as_uint(a[i + 2]), false, false);
    b[i] = __uint_as_float(p.x) + __uint_as_float(p.y);
  }
  // 8-lane halves of a row (mirror pairing): lanes 0-7 keep b[0], 8-15 b[1]
  const bool upper = lane & 8;
  const float keep = upper ? b[1] : b[0], give = upper ? b[0] : b[1];
  float r = keep + dpp_f<kDppMirror>(give);
  r += dpp_f<kDppXor1>(r);
  r += dpp_f<kDppXor2>(r);
  r += dpp_f<kDppHalfMirror>(r);
  return r;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  u32x2_t p = swap16(__float_as_uint(v));
  v = fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
  p = swap32(__float_as_uint(v));
  return fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  u32x2_t p = swap16(v);
  v = max(p.x, p.y);
  p = swap32(v);
  return max(p.x, p.y);
}

// Order-preserving map of a float to an unsigned (larger float, larger key;
// -0 sorts just below +0).
__device__ __forceinline__ uint32_t ordered_bits(float z) {
  const uint32_t b = __float_as_uint(z);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// (value, index) maximum over the wave: larger value, then smaller index.
// Values must not be NaN.  Every lane receives the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  const float m = wave_max(v);
  // lowest index among the lanes holding the maximum
  const int cand = v == m ? i : 0x7FFFFFFF;
  uint32_t c = (uint32_t)cand;
  c = min(c, dpp_u<kDppXor1>(c));
  c = min(c, dpp_u<kDppXor2>(c));
  c = min(c, dpp_u<kDppHalfMirror>(c));
  c = min(c, dpp_u<kDppMirror>(c));
  u32x2_t p = swap16(c);
  c = min(p.x, p.y);
  p = swap32(c);
  c = min(p.x, p.y);
  v = m;
  i = (int)c;
}

// ---- cross-workgroup hand-off without cache maintenance -------------------
// Data that other workgroups read during the same kernel is written and read
// with agent-scope relaxed atomics (global_store/load with sc1: coherent
// across the XCDs' L2s), so no L2 writeback or invalidate is needed.  The
// writer waits for its stores to complete before bumping the arrival
// counter; the reader issues its loads only after it has seen the count.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long load_coherent(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// All of this wave's outstanding memory operations have completed.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ unsigned arrive(unsigned* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Activation range.  Activations reach binary16 operands (the batched
// kernels' x, and h on every path) scaled by a power of two: x 2^a with a
// chosen from the row's largest magnitude, so that it lies in [1, 2).  Then
// g and u carry 2^a, h = w silu(g) u is formed as 2^(2a) h, and the output
// is scaled back by 2^(-2a); all scalings are exact, so any bf16 magnitude
// works (h 2^(2a) is bounded by the weights alone).
// The larger magnitude (bits, sign cleared) of a dword's two bf16 values.
__device__ __forceinline__ uint32_t bf16_mag_max(uint32_t w) { return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu); }
// a for a row whose largest magnitude has bf16 bits mb (sign cleared): 127
// minus its biased exponent, within [-126, 126]; 0 for an all-zero row.
__device__ __forceinline__ int act_exponent(uint32_t mb) {
  if (mb == 0u) return 0;
  return min(max(127 - (int)(mb >> 7), -126), 126);
}
// 2^a silu(g) from g (exact scaling of the quotient).
__device__ __forceinline__ float silu_scaled(float g, int a) { return ldexpf(g, a) / (1.0f + expf(-g)); }

// Byte offset, within its matrix, of the 16-byte piece c of row r.
__device__ __forceinline__ size_t piece_offset(size_t row, int pieces_per_row, int c) {
  return (row * (size_t)pieces_per_row + (size_t)c) * 16u;
}

}  // namespace moe
