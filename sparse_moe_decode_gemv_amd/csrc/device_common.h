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

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (b >> 16) | 0x40u;  // quiet NaN
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

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
  s.p0 = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[4]) << 16);
  s.p1 = f32_to_bf16_bits(v[1] * 0.125f) | (f32_to_bf16_bits(v[5] * 0.125f) << 16);
  s.p2 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[6]) << 16);
  s.p3 = f32_to_bf16_bits(v[3] * 0.125f) | (f32_to_bf16_bits(v[7] * 0.125f) << 16);
  s.corr = -136.0f * ((v[0] + v[4]) + (v[2] + v[6])) - 24.0f * ((v[1] + v[5]) + (v[3] + v[7]));
  return s;
}

// From 8 bf16 values held as 4 dwords (dword i = elements 2i (low), 2i+1 (high)).
__device__ __forceinline__ Slice8 make_slice_bf16(uint4 q) {
  float v[8];
  v[0] = bf16_bits_to_f32(q.x & 0xFFFFu);
  v[1] = bf16_bits_to_f32(q.x >> 16);
  v[2] = bf16_bits_to_f32(q.y & 0xFFFFu);
  v[3] = bf16_bits_to_f32(q.y >> 16);
  v[4] = bf16_bits_to_f32(q.z & 0xFFFFu);
  v[5] = bf16_bits_to_f32(q.z >> 16);
  v[6] = bf16_bits_to_f32(q.w & 0xFFFFu);
  v[7] = bf16_bits_to_f32(q.w >> 16);
  return make_slice(v);
}

// fp32 activations split as hi = bf16(v), lo = bf16(v - hi): two slices whose
// sum carries v to about 2^-16 relative.
__device__ __forceinline__ void make_slice_hilo(const float v[8], Slice8& hi, Slice8& lo) {
  float h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = bf16_bits_to_f32(f32_to_bf16_bits(v[e]));
    l[e] = bf16_bits_to_f32(f32_to_bf16_bits(v[e] - h[e]));
  }
  hi = make_slice(h);
  lo = make_slice(l);
}

// acc + sum_e (128+u_e or 128+8u_e) * (x_e or x_e/8); started from s.corr
// this is sum_e (u_e - 8) x_e.
__device__ __forceinline__ float dot8(uint32_t w, const Slice8& s, float acc) {
  acc = dot2_bf16((w & 0x000F000Fu) | 0x43004300u, s.p0, acc);
  acc = dot2_bf16(((w >> 1) & 0x00780078u) | 0x43004300u, s.p1, acc);
  acc = dot2_bf16(((w >> 8) & 0x000F000Fu) | 0x43004300u, s.p2, acc);
  acc = dot2_bf16(((w >> 9) & 0x00780078u) | 0x43004300u, s.p3, acc);
  return acc;
}

// One 16-byte piece (4 groups x 8 codes) against 4 prepared slices, scaled by
// the 4 groups' binary16 scales (sc.x = groups 0,1; sc.y = groups 2,3).
__device__ __forceinline__ float dot_piece(uint4 q, const Slice8 xs[4], uint2 sc) {
  float p = dot8(q.x, xs[0], xs[0].corr) * f16_bits_to_f32(sc.x & 0xFFFFu);
  p = fmaf(dot8(q.y, xs[1], xs[1].corr), f16_bits_to_f32(sc.x >> 16), p);
  p = fmaf(dot8(q.z, xs[2], xs[2].corr), f16_bits_to_f32(sc.y & 0xFFFFu), p);
  p = fmaf(dot8(q.w, xs[3], xs[3].corr), f16_bits_to_f32(sc.y >> 16), p);
  return p;
}

__device__ __forceinline__ float dot_piece_hilo(uint4 q, const Slice8 hi[4], const Slice8 lo[4], uint2 sc) {
  float p = dot8(q.x, lo[0], dot8(q.x, hi[0], hi[0].corr + lo[0].corr)) * f16_bits_to_f32(sc.x & 0xFFFFu);
  p = fmaf(dot8(q.y, lo[1], dot8(q.y, hi[1], hi[1].corr + lo[1].corr)), f16_bits_to_f32(sc.x >> 16), p);
  p = fmaf(dot8(q.z, lo[2], dot8(q.z, hi[2], hi[2].corr + lo[2].corr)), f16_bits_to_f32(sc.y & 0xFFFFu), p);
  p = fmaf(dot8(q.w, lo[3], dot8(q.w, hi[3], hi[3].corr + lo[3].corr)), f16_bits_to_f32(sc.y >> 16), p);
  return p;
}

// Sum over aligned segments of SEG lanes (SEG a power of two <= 64); every
// lane of a segment receives the segment's sum.
template <int SEG>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
  for (int o = SEG / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return seg_sum<64>(v); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Byte offset, within its matrix, of the 16-byte piece c of row r.
__device__ __forceinline__ size_t piece_offset(size_t row, int pieces_per_row, int c) {
  return (row * (size_t)pieces_per_row + (size_t)c) * 16u;
}

}  // namespace moe
