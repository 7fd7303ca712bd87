// lmhead.cpp -- plain, slow fp64 C++ oracle of the 4-bit output layer (LM
// head) with argmax.
//
// TEST INFRASTRUCTURE ONLY: part of the plain CPU oracle; shares no code with
// the GPU path.
//
// The pages state that the output layer maps the hidden state back to a
// vocabulary of about 150,000 tokens, costs about an eighth of the per-token
// work and is quantized to 4 bits ("Flint 40B: Best Mid Sized LLM",
// transcript 03:36-05:39; mirrorspeed.com page, section "Quantization").
// Decoding here is greedy: the token is the index of the largest logit, the
// lowest index on ties.  Weights are int4 with one binary16 scale per 32
// elements, stored as in formats.h.
#include <cstdint>
#include <vector>

#include "formats.h"

extern "C" {

// z[b][v] = sum_k W[v][k] x[b][k] in fp64 for B bf16 rows x; tok[b] the
// first v reaching the row's maximum, zmax[b] that maximum; z (B x V) is
// written when not NULL.
void orc_lmhead(const uint8_t* wq, const uint16_t* ws, int V, int d, const uint16_t* x_bits, int B, int32_t* tok,
                double* zmax, double* z) {
  std::vector<double> x((size_t)B * d);
  for (size_t i = 0; i < x.size(); ++i) x[i] = orc::bf16_to_f64(x_bits[i]);
  std::vector<double> zz((size_t)B * V);
#pragma omp parallel
  {
    std::vector<double> w(d);
#pragma omp for schedule(static)
    for (int v = 0; v < V; ++v) {
      const uint8_t* qr = wq + (size_t)v * (d / 2);
      for (int k = 0; k < d; ++k)
        w[k] = (double)(orc::code_at(qr, k) - 8) * orc::f16_to_f64(ws[(size_t)v * (d / 32) + k / 32]);
      for (int b = 0; b < B; ++b) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += w[k] * x[(size_t)b * d + k];
        zz[(size_t)b * V + v] = acc;
      }
    }
  }
  for (int b = 0; b < B; ++b) {
    int best = 0;
    for (int v = 1; v < V; ++v)
      if (zz[(size_t)b * V + v] > zz[(size_t)b * V + best]) best = v;
    tok[b] = best;
    zmax[b] = zz[(size_t)b * V + best];
    if (z)
      for (int v = 0; v < V; ++v) z[(size_t)b * V + v] = zz[(size_t)b * V + v];
  }
}

}  // extern "C"
