/*
 * synth.c -- seeded synthetic inputs shared by the tests and the benchmark.
 *
 * Holds only the input recipe: a counter-based random stream, normal draws,
 * fp32->bf16 rounding of activations, and the offline int4 quantize-and-pack
 * step that turns fp32 weight draws into the library's stored weight format.
 * None of the decode step's arithmetic (router, softmax, top-k, expert GEMVs,
 * combine, LM head) lives here.
 *
 * Random stream: SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used in counter mode: value i
 * of a stream with key K is the SplitMix64 output mix(K + (i+1)*GAMMA).  Any
 * element can be regenerated on its own, so the output does not depend on the
 * number of threads.  Normals come from the Box-Muller transform (Box &
 * Muller, 1958): one 64-bit stream value gives two 24-bit uniforms and
 * thereby one (r cos, r sin) pair, in single precision (normal.c).
 *
 * int4 weight format (K a multiple of 128, rows stored one after another,
 * K/2 bytes per row):
 *   element k of a row:  t = k/128, j = (k%128)/32, q = (k%32)/8, e = k%8
 *   byte within the row: 64*t + 16*q + 4*j + e/2
 *   nibble:              low 4 bits when e is even, high 4 bits when e is odd
 *   stored code u in [0,15]; the weight is (u - 8) * scale[row][k/32]
 *   scales: IEEE binary16 bits, [rows][K/32] row-major.
 * Quantizer for one group of 32 fp32 values w: a = max|w|,
 * s = fp16_rne(a/7) with a/7 taken in fp64; s == 0 gives q = 0 everywhere,
 * otherwise q = clamp(round_half_even(w/s), -7, 7); u = q + 8.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Value i of the stream keyed by `key`. */
static inline uint64_t stream_u64(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GAMMA);
}


uint64_t synth_key(uint64_t parent, uint64_t tag) {
  return mix64(mix64(parent ^ 0x632BE59BD9B4E019ull) + (tag + 1) * GAMMA);
}

uint64_t synth_u64(uint64_t key, uint64_t i) { return stream_u64(key, i); }

void synth_normal_block16(uint64_t key, uint64_t p0, float* a, float* b);

/* 32 consecutive standard normals starting at element 32*blk: element 2p is
 * the cosine half and element 2p+1 the sine half of pair p. */
static inline void normal_block32(uint64_t key, uint64_t blk, float* out) {
  float a[16], b[16];
  synth_normal_block16(key, blk * 16, a, b);
  for (int i = 0; i < 16; ++i) {
    out[2 * i] = a[i];
    out[2 * i + 1] = b[i];
  }
}

static inline uint16_t f32_to_bf16_rne(float v) {
  uint32_t b;
  memcpy(&b, &v, 4);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (uint16_t)((b >> 16) | 0x40);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* fp64 -> IEEE binary16, round to nearest even (subnormals and overflow
 * handled); relies on the default rounding mode for nearbyint(). */
static uint16_t f64_to_f16_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return sign | 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;
  if (a < 0x1p-14) return sign | (uint16_t)nearbyint(a * 0x1p24);
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  double r = nearbyint(ldexp(a, 11 - e)); /* [1024, 2048] */
  int ex = e - 1;
  if (r == 2048.0) { r = 1024.0; ex += 1; }
  if (ex > 15) return sign | 0x7C00;
  return sign | (uint16_t)(((ex + 15) << 10) | ((int)r - 1024));
}

static double f16_value(uint16_t h) {
  int ex = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v = ex == 0 ? ldexp((double)m, -24) : ldexp((double)(m + 1024), ex - 25);
  return (h & 0x8000) ? -v : v;
}

static inline int64_t packed_offset(int64_t k) {
  int64_t t = k >> 7, j = (k >> 5) & 3, q = (k >> 3) & 3, e = k & 7;
  return 64 * t + 16 * q + 4 * j + (e >> 1);
}

/* Quantize one group of 32 values; writes codes u[32] and returns scale bits. */
static uint16_t quantize_group(const float* w, uint8_t* u) {
  float a = 0.f;
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(w[i]));
  uint16_t sb = f64_to_f16_rne((double)a / 7.0);
  double s = f16_value(sb);
  for (int i = 0; i < 32; ++i) {
    if (s == 0.0) { u[i] = 8; continue; }
    double q = nearbyint((double)w[i] / s);
    if (q > 7) q = 7;
    if (q < -7) q = -7;
    u[i] = (uint8_t)(q + 8);
  }
  return sb;
}

/* MXFP4 block of 32 (the OCP MX v1.0 conversion): shared exponent
 * X = floor(log2 amax) - 2 (2: the largest E2M1 exponent), scale byte
 * X + 127 kept in 0..254; each |w| / 2^X goes to the nearest E2M1 magnitude
 * (0, 0.5, 1, 1.5, 2, 3, 4, 6), a tie to the even code, anything above 6 to
 * 6, the sign into bit 3 (zero stays code 0).  An all-zero block gets scale
 * byte 127 and codes 0.  Writes codes u[32], returns the scale byte. */
static uint8_t quantize_group_mxfp4(const float* w, uint8_t* u) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  float a = 0.f;
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(w[i]));
  if (a == 0.f) {
    memset(u, 0, 32);
    return 127;
  }
  int e;
  frexp((double)a, &e); /* a = m 2^e, 0.5 <= m < 1: floor(log2 a) = e - 1 */
  int b = e - 1 - 2 + 127;
  if (b < 0) b = 0;
  if (b > 254) b = 254;
  const double sc = ldexp(1.0, b - 127);
  for (int i = 0; i < 32; ++i) {
    const double v = fabs((double)w[i]) / sc;
    int best = 0;
    double bd = v;
    for (int c = 1; c < 8; ++c) {
      const double dd = fabs(v - mag[c]);
      if (dd < bd || (dd == bd && (c & 1) == 0 && (best & 1) != 0)) {
        best = c;
        bd = dd;
      }
    }
    u[i] = (uint8_t)(best | (w[i] < 0.f && best > 0 ? 8 : 0));
  }
  return (uint8_t)b;
}

static void pack_row(const uint8_t* u, int64_t K, uint8_t* row) {
  memset(row, 0, (size_t)(K / 2));
  for (int64_t k = 0; k < K; ++k) {
    int64_t o = packed_offset(k);
    row[o] |= (uint8_t)((k & 1) ? (u[k] << 4) : u[k]);
  }
}

void synth_normal_f32(float* out, int64_t n, uint64_t key, double mu, double sigma) {
#pragma omp parallel for schedule(static)
  for (int64_t blk = 0; blk < (n + 31) / 32; ++blk) {
    float z[32];
    normal_block32(key, (uint64_t)blk, z);
    for (int i = 0; i < 32 && blk * 32 + i < n; ++i) out[blk * 32 + i] = (float)(mu + sigma * (double)z[i]);
  }
}

void synth_bf16(uint16_t* out, int64_t n, uint64_t key, double mu, double sigma) {
#pragma omp parallel for schedule(static)
  for (int64_t blk = 0; blk < (n + 31) / 32; ++blk) {
    float z[32];
    normal_block32(key, (uint64_t)blk, z);
    for (int i = 0; i < 32 && blk * 32 + i < n; ++i)
      out[blk * 32 + i] = f32_to_bf16_rne((float)(mu + sigma * (double)z[i]));
  }
}

/* Weight matrix [rows][K] with N(0, sigma) fp32 entries (element r*K+k of
 * the stream), quantized per group of 32 and packed.  w_out (may be NULL)
 * receives the fp32 draws, for checking the quantizer. */
void synth_int4(uint8_t* q, uint16_t* s, int64_t rows, int64_t K, uint64_t key, double sigma, float* w_out) {
#pragma omp parallel
  {
    float w[32];
    uint8_t u[32];
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      uint8_t* row = q + r * (K / 2);
      memset(row, 0, (size_t)(K / 2));
      for (int64_t g = 0; g < K / 32; ++g) {
        normal_block32(key, (uint64_t)(r * (K / 32) + g), w);
        for (int i = 0; i < 32; ++i) w[i] = (float)(sigma * (double)w[i]);
        if (w_out) memcpy(w_out + r * K + g * 32, w, sizeof w);
        s[r * (K / 32) + g] = quantize_group(w, u);
        for (int i = 0; i < 32; ++i) {
          int64_t k = g * 32 + i;
          row[packed_offset(k)] |= (uint8_t)((k & 1) ? (u[i] << 4) : u[i]);
        }
      }
    }
  }
}

/* E matrices [rows][K], matrix e drawn from stream synth_key(key, e). */
void synth_int4_experts(uint8_t* q, uint16_t* s, int64_t E, int64_t rows, int64_t K, uint64_t key, double sigma) {
#pragma omp parallel
  {
    float w[32];
    uint8_t u[32];
#pragma omp for schedule(static) collapse(2)
    for (int64_t e = 0; e < E; ++e)
      for (int64_t r = 0; r < rows; ++r) {
        uint64_t ek = synth_key(key, (uint64_t)e);
        int64_t rr = e * rows + r;
        uint8_t* row = q + rr * (K / 2);
        memset(row, 0, (size_t)(K / 2));
        for (int64_t g = 0; g < K / 32; ++g) {
          normal_block32(ek, (uint64_t)(r * (K / 32) + g), w);
          for (int i = 0; i < 32; ++i) w[i] = (float)(sigma * (double)w[i]);
          s[rr * (K / 32) + g] = quantize_group(w, u);
          for (int i = 0; i < 32; ++i) {
            int64_t k = g * 32 + i;
            row[packed_offset(k)] |= (uint8_t)((k & 1) ? (u[i] << 4) : u[i]);
          }
        }
      }
  }
}

/* Quantize and pack caller-given fp32 weights [rows][K]. */
void synth_quantize_pack(const float* w, int64_t rows, int64_t K, uint8_t* q, uint16_t* s) {
#pragma omp parallel
  {
    uint8_t u[32];
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      uint8_t* row = q + r * (K / 2);
      memset(row, 0, (size_t)(K / 2));
      for (int64_t g = 0; g < K / 32; ++g) {
        s[r * (K / 32) + g] = quantize_group(w + r * K + g * 32, u);
        for (int i = 0; i < 32; ++i) {
          int64_t k = g * 32 + i;
          row[packed_offset(k)] |= (uint8_t)((k & 1) ? (u[i] << 4) : u[i]);
        }
      }
    }
  }
}

/* Pack caller-given codes u[rows][K] (values 0..15) into the stored layout. */
void synth_pack_codes(const uint8_t* u, int64_t rows, int64_t K, uint8_t* q) {
  for (int64_t r = 0; r < rows; ++r) pack_row(u + r * K, K, q + r * (K / 2));
}

/* Fisher-Yates shuffle of 0..n-1 driven by the stream. */
void synth_permutation(int32_t* out, int32_t n, uint64_t key) {
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    uint64_t j = stream_u64(key, (uint64_t)i) % (uint64_t)(i + 1);
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/* MXFP4 counterparts: E matrices [rows][K] from the same streams as
 * synth_int4_experts, E2M1 codes packed at the same nibble positions, one
 * E8M0 scale byte per 32 elements. */
void synth_mxfp4_experts(uint8_t* q, uint8_t* s, int64_t E, int64_t rows, int64_t K, uint64_t key, double sigma) {
#pragma omp parallel
  {
    float w[32];
    uint8_t u[32];
#pragma omp for schedule(static) collapse(2)
    for (int64_t e = 0; e < E; ++e)
      for (int64_t r = 0; r < rows; ++r) {
        uint64_t ek = synth_key(key, (uint64_t)e);
        int64_t rr = e * rows + r;
        uint8_t* row = q + rr * (K / 2);
        memset(row, 0, (size_t)(K / 2));
        for (int64_t g = 0; g < K / 32; ++g) {
          normal_block32(ek, (uint64_t)(r * (K / 32) + g), w);
          for (int i = 0; i < 32; ++i) w[i] = (float)(sigma * (double)w[i]);
          s[rr * (K / 32) + g] = quantize_group_mxfp4(w, u);
          for (int i = 0; i < 32; ++i) {
            int64_t k = g * 32 + i;
            row[packed_offset(k)] |= (uint8_t)((k & 1) ? (u[i] << 4) : u[i]);
          }
        }
      }
  }
}

void synth_quantize_pack_mxfp4(const float* w, int64_t rows, int64_t K, uint8_t* q, uint8_t* s) {
#pragma omp parallel
  {
    uint8_t u[32];
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      uint8_t* row = q + r * (K / 2);
      memset(row, 0, (size_t)(K / 2));
      for (int64_t g = 0; g < K / 32; ++g) {
        s[r * (K / 32) + g] = quantize_group_mxfp4(w + r * K + g * 32, u);
        for (int i = 0; i < 32; ++i) {
          int64_t k = g * 32 + i;
          row[packed_offset(k)] |= (uint8_t)((k & 1) ? (u[i] << 4) : u[i]);
        }
      }
    }
  }
}

/* Nearest E2M1 code of a magnitude v >= 0 (ties to the even code, above 6
 * to 6). */
static int e2m1_nearest(double v) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  int best = 0;
  double bd = v;
  for (int c = 1; c < 8; ++c) {
    const double dd = fabs(v - mag[c]);
    if (dd < bd || (dd == bd && (c & 1) == 0 && (best & 1) != 0)) {
      best = c;
      bd = dd;
    }
  }
  return best;
}

/* Nearest OCP E4M3FN byte of x >= 0 (ties to even, at most 448 = 0x7E):
 * x = m 2^e with 0.5 <= m < 1 has exponent field e + 6 when that is >= 1
 * (mantissa (2m - 1) * 8 rounded), else it is a subnormal x / 2^-9. */
static uint8_t e4m3_nearest(double x) {
  if (!(x > 0.0)) return 0;
  if (x >= 448.0) return 0x7E;
  int e;
  const double m = frexp(x, &e);
  int E = e + 6;
  if (E < 1) return (uint8_t)nearbyint(x * 512.0); /* 0..8; 8 is the smallest normal */
  double mant = nearbyint((2.0 * m - 1.0) * 8.0);
  if (mant >= 8.0) {
    mant = 0.0;
    ++E;
  }
  if (E > 15 || (E == 15 && mant >= 7.0)) return 0x7E;
  return (uint8_t)((E << 3) | (int)mant);
}

static double e4m3_value(uint8_t b) {
  const int E = (b >> 3) & 15, m = b & 7;
  return E == 0 ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, E - 7);
}

/* NVFP4 of one matrix [rows][K] (two-level: an fp32 tensor scale
 * amax / (6 * 448), an E4M3 scale per 16 elements nearest to
 * amax(block) / 6 / t, E2M1 codes nearest to w / (e4m3 * t)); returns t. */
static float quantize_matrix_nvfp4(const float* w, int64_t rows, int64_t K, uint8_t* q, uint8_t* s) {
  float amax = 0.f;
  for (int64_t i = 0; i < rows * K; ++i) amax = fmaxf(amax, fabsf(w[i]));
  const float t = (float)((double)amax / (6.0 * 448.0));
  memset(q, 0, (size_t)(rows * K / 2));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < K / 16; ++b) {
      const float* x = w + r * K + b * 16;
      float ab = 0.f;
      for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(x[i]));
      const uint8_t sb = t > 0.f ? e4m3_nearest((double)ab / 6.0 / (double)t) : 0;
      s[r * (K / 16) + b] = sb;
      const double sc = e4m3_value(sb) * (double)t;
      for (int i = 0; i < 16; ++i) {
        const int c0 = sc > 0.0 ? e2m1_nearest(fabs((double)x[i]) / sc) : 0;
        const int c = c0 | (x[i] < 0.f && c0 > 0 ? 8 : 0);
        const int64_t k = b * 16 + i;
        q[r * (K / 2) + packed_offset(k)] |= (uint8_t)((k & 1) ? (c << 4) : c);
      }
    }
  return t;
}

/* E NVFP4 matrices [rows][K] from the same streams as synth_int4_experts. */
void synth_nvfp4_experts(uint8_t* q, uint8_t* s, float* t, int64_t E, int64_t rows, int64_t K, uint64_t key,
                         double sigma) {
#pragma omp parallel
  {
    float* w = (float*)malloc((size_t)(rows * K) * sizeof(float));
#pragma omp for schedule(static)
    for (int64_t e = 0; e < E; ++e) {
      const uint64_t ek = synth_key(key, (uint64_t)e);
      for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < K / 32; ++g) {
          float z[32];
          normal_block32(ek, (uint64_t)(r * (K / 32) + g), z);
          for (int i = 0; i < 32; ++i) w[r * K + g * 32 + i] = (float)(sigma * (double)z[i]);
        }
      t[e] = quantize_matrix_nvfp4(w, rows, K, q + e * rows * (K / 2), s + e * rows * (K / 16));
    }
    free(w);
  }
}

float synth_quantize_nvfp4(const float* w, int64_t rows, int64_t K, uint8_t* q, uint8_t* s) {
  return quantize_matrix_nvfp4(w, rows, K, q, s);
}
