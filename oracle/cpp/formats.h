// formats.h -- number formats of the decode path, decoded from their bit
// fields in fp64 (plain C++ oracle).
//
// TEST INFRASTRUCTURE ONLY: part of the plain CPU oracle.  Nothing in the
// product path may include, link or call this; it shares no code with the
// GPU kernels.
//
// The pages say the model ships 4-bit ("int4") builds and a 4-bit output
// layer ("Flint 40B: Best Mid Sized LLM", transcript 05:39 and 07:15) and
// name NVFP4 for the released model ("Recursive Releases Flint...", section
// "Quantization"); they fix no group size, scale type or nibble order.  The
// stored formats read here are the stated choices of this project:
//
//   int4   code u in 0..15, weight (u - 8) * s, one IEEE binary16 scale s
//          per 32 consecutive elements along K;
//   MXFP4  FP4 E2M1 code, one E8M0 scale byte (2^(b - 127)) per 32;
//   NVFP4  FP4 E2M1 code, one OCP E4M3FN scale byte per 16 and one fp32
//          scale per expert matrix.
//
// Element k of a stored row (K a multiple of 128) is the nibble of byte
// 64 t + 16 q + 4 j + e/2 with t = k/128, j = (k%128)/32, q = (k%32)/8,
// e = k%8: the low nibble for even e, the high one for odd e.
#pragma once

#include <cmath>
#include <cstdint>
#include <cstring>

namespace orc {

// bfloat16: the upper half of an IEEE binary32.
inline double bf16_to_f64(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
inline double f16_to_f64(uint16_t b) {
  const double sign = (b & 0x8000u) ? -1.0 : 1.0;
  const int ex = (b >> 10) & 0x1F, fr = b & 0x3FF;
  if (ex == 0) return sign * std::ldexp((double)fr, -24);            // fr/1024 * 2^-14
  if (ex == 31) return fr ? NAN : sign * INFINITY;
  return sign * std::ldexp(1024.0 + fr, ex - 25);                     // (1 + fr/1024) 2^(ex-15)
}

// FP4 E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.
inline double e2m1_to_f64(int c) {
  const double sign = (c & 8) ? -1.0 : 1.0;
  const int ex = (c >> 1) & 3, m = c & 1;
  return sign * (ex == 0 ? 0.5 * m : std::ldexp(2.0 + m, ex - 2));    // (1 + m/2) 2^(ex-1)
}

// E8M0: 2^(b - 127); b = 255 is NaN.
inline double e8m0_to_f64(uint8_t b) { return b == 255 ? NAN : std::ldexp(1.0, (int)b - 127); }

// OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no
// infinity, S.1111.111 is NaN.
inline double e4m3_to_f64(uint8_t b) {
  if ((b & 0x7F) == 0x7F) return NAN;
  const double sign = (b & 0x80) ? -1.0 : 1.0;
  const int ex = (b >> 3) & 0xF, m = b & 7;
  return sign * (ex == 0 ? std::ldexp((double)m, -9) : std::ldexp(8.0 + m, ex - 10));  // m/8 2^-6 | (1+m/8) 2^(ex-7)
}

// Stored 4-bit code of element k of a row.
inline int code_at(const uint8_t* row, int k) {
  const int t = k / 128, j = (k % 128) / 32, q = (k % 32) / 8, e = k % 8;
  return (row[64 * t + 16 * q + 4 * j + e / 2] >> (4 * (e & 1))) & 0xF;
}

// fp64 -> bfloat16 bits, round to nearest, ties to even (finite inputs).
inline uint16_t f64_to_bf16(double x) {
  double y;
  if (x == 0.0 || std::fabs(x) < std::ldexp(1.0, -126)) {
    y = std::ldexp(std::nearbyint(std::ldexp(x, 133)), -133);  // subnormal quantum 2^-133
  } else {
    int e;
    const double m = std::frexp(x, &e);                         // x = m 2^e, 0.5 <= |m| < 1
    y = std::ldexp(std::nearbyint(m * 256.0) / 256.0, e);       // 8 significant bits
  }
  const float f = (float)y;                                     // exact
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

// fp64 -> binary16 bits, round to nearest, ties to even; overflow to inf.
inline uint16_t f64_to_f16(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
  const double a = std::fabs(x);
  if (a != a) return 0x7E00u;
  if (a < std::ldexp(1.0, -14)) {                      // subnormal: quantum 2^-24
    const double q = std::nearbyint(std::ldexp(a, 24));  // 1024 is the smallest normal, same bits
    return (uint16_t)(sign | (uint16_t)q);
  }
  int e;
  double m = std::frexp(a, &e);                        // a = m 2^e
  double r = std::nearbyint(m * 2048.0);               // 11 significant bits, 1024..2048
  if (r == 2048.0) {
    r = 1024.0;
    ++e;
  }
  const int field = e - 1 + 15;                        // a = (r / 1024) 2^(e - 1)
  if (field >= 31) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)(field << 10) | (uint16_t)(r - 1024.0));
}

}  // namespace orc
