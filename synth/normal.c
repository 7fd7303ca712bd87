/*
 * normal.c -- Box-Muller normal draws for synth.c, 16 pairs at a time.
 *
 * Compiled on its own with -O3 -ffast-math so that the float log/cos/sin
 * loops use glibc's vector math; the shared library is linked without
 * -ffast-math, so loading it does not change the process's floating-point
 * modes.  Values depend only on (key, pair index), never on the thread that
 * computes them.
 */
#include <math.h>
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Standard normal pairs p0 .. p0+15 of the stream `key`: stream value p (the
 * SplitMix64 output mix(key + (p+1)*GAMMA)) gives two 24-bit uniforms on
 * (0, 1]; a[i] = r cos(theta), b[i] = r sin(theta). */
void synth_normal_block16(uint64_t key, uint64_t p0, float* a, float* b) {
  int32_t h[16], l[16];
  float r[16], th[16];
  for (int i = 0; i < 16; ++i) {
    uint64_t x = mix64(key + (p0 + (uint64_t)i + 1) * GAMMA);
    h[i] = (int32_t)(x >> 40);
    l[i] = (int32_t)((x >> 8) & 0xFFFFFF);
  }
#pragma omp simd
  for (int i = 0; i < 16; ++i) {
    r[i] = sqrtf(-2.0f * logf(((float)h[i] + 1.0f) * 0x1p-24f));
    th[i] = 6.2831853071795865f * (((float)l[i] + 1.0f) * 0x1p-24f);
  }
#pragma omp simd
  for (int i = 0; i < 16; ++i) a[i] = r[i] * cosf(th[i]);
#pragma omp simd
  for (int i = 0; i < 16; ++i) b[i] = r[i] * sinf(th[i]);
}
