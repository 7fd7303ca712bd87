// moe.cpp -- plain, slow fp64 C++ oracle of one sparse MoE layer decode step
// and of the pre-norm stack of such layers.
//
// TEST INFRASTRUCTURE ONLY: part of the plain CPU oracle.  Only the tests,
// the smoke check and the CPU-baseline leg of the benchmark load it; it
// shares no code with the GPU path (its own decoders in formats.h, its own
// loops) and the product path never links it.
//
// What the pages fix ("Flint 40B: Best Mid Sized LLM", transcript 02:35):
// every MoE layer holds 256 routed experts, a small router picks a few per
// token and only those run; the pages' own layer adds one always-on shared
// expert.  What they leave open is read as follows:
//
//   router   l_e = sum_k W_r[e][k] x_k + b_e in fp64 (fp32 weights, bf16 x);
//   select   the k largest logits, ties to the lower expert index (the
//            softmax is strictly increasing, so these are the k largest
//            probabilities); p = softmax(l) over all E experts; the weights
//            are p renormalized over the chosen set (norm = 1) or p itself;
//   expert   SwiGLU: h_i = silu(g_i) u_i with g = W_g x, u = W_u x and
//            silu(z) = z / (1 + e^-z), then o = W_d h, all on dequantized
//            4-bit weights in fp64;
//   combine  y = sum of w_j o_j over the chosen experts in ascending expert
//            index; a shared expert's output is added after, weight 1;
//   stack    r_0 = fp32(x_0); x_l = bf16(r_l / sqrt(mean(r_l^2) + eps)),
//            y_l = layer(x_l) rounded to fp32, r_{l+1} = fp32(r_l + y_l).
//
// Every loop is the definition written out: one dot product per output
// element, summed in index order, so the result does not depend on the
// number of OpenMP threads (the threads split output rows only).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <thread>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

#include "formats.h"

extern "C" {

// One stored 4-bit matrix family: codes [n][rows][K/2], scales and, for
// NVFP4, fp32 matrix scales [n] (n = E, or 1 for the shared expert).
struct orc_mat {
  const uint8_t* q;
  const void* s;
  const float* ts;
};

// One layer.  fmt: 0 int4 (binary16 scale per 32), 1 MXFP4 (E8M0 per 32),
// 2 NVFP4 (E4M3 per 16, fp32 per matrix).
struct orc_layer {
  int32_t d, f, E, fmt, has_shared, pad;
  const float* router_w;  // [E][d]
  const float* router_b;  // [E] or NULL
  orc_mat gate, up, down;            // [E][f][d], [E][f][d], [E][d][f] (element counts)
  orc_mat sh_gate, sh_up, sh_down;   // the shared expert, when has_shared
};

}  // extern "C"

namespace {

// Row r of matrix n (rows x K elements) of a family, dequantized into w[K].
void dequant_row(const orc_mat& m, int fmt, size_t n, size_t rows, int K, size_t r, double* w) {
  const size_t row = n * rows + r;
  const uint8_t* qr = m.q + row * (size_t)(K / 2);
  for (int k = 0; k < K; ++k) {
    const int c = orc::code_at(qr, k);
    if (fmt == 0) {
      const uint16_t s = static_cast<const uint16_t*>(m.s)[row * (size_t)(K / 32) + k / 32];
      w[k] = (double)(c - 8) * orc::f16_to_f64(s);
    } else if (fmt == 1) {
      const uint8_t s = static_cast<const uint8_t*>(m.s)[row * (size_t)(K / 32) + k / 32];
      w[k] = orc::e2m1_to_f64(c) * orc::e8m0_to_f64(s);
    } else {
      const uint8_t s = static_cast<const uint8_t*>(m.s)[row * (size_t)(K / 16) + k / 16];
      w[k] = orc::e2m1_to_f64(c) * orc::e4m3_to_f64(s) * (double)m.ts[n];
    }
  }
}

// out[r] = sum_k W[r][k] v[k] for the rows of matrix n of a family.
void matvec(const orc_mat& m, int fmt, size_t n, int rows, int K, const double* v, double* out) {
#pragma omp parallel
  {
    std::vector<double> w(K);
#pragma omp for schedule(static)
    for (int r = 0; r < rows; ++r) {
      dequant_row(m, fmt, n, rows, K, r, w.data());
      double acc = 0.0;
      for (int k = 0; k < K; ++k) acc += w[k] * v[k];
      out[r] = acc;
    }
  }
}

// o = W_d (silu(W_g x) * (W_u x)) of expert n of the given families.
void expert_forward(const orc_layer* L, const orc_mat& g, const orc_mat& u, const orc_mat& dn, size_t n,
                    const double* x, double* o) {
  const int d = L->d, f = L->f;
  std::vector<double> gv(f), uv(f), h(f);
  matvec(g, L->fmt, n, f, d, x, gv.data());
  matvec(u, L->fmt, n, f, d, x, uv.data());
  for (int i = 0; i < f; ++i) h[i] = gv[i] / (1.0 + std::exp(-gv[i])) * uv[i];
  matvec(dn, L->fmt, n, d, f, h.data(), o);
}

void router(const orc_layer* L, const double* x, double* l) {
  const int E = L->E, d = L->d;
#pragma omp parallel for schedule(static)
  for (int e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int k = 0; k < d; ++k) acc += (double)L->router_w[(size_t)e * d + k] * x[k];
    l[e] = acc + (L->router_b ? (double)L->router_b[e] : 0.0);
  }
}

void to_f64(const uint16_t* bits, int n, double* out) {
  for (int i = 0; i < n; ++i) out[i] = orc::bf16_to_f64(bits[i]);
}

}  // namespace

extern "C" {

int orc_abi_version(void) { return 1; }

// Threads the oracle's loops may use (1 = single-threaded), and the host's
// hardware thread count.
void orc_set_threads(int n) {
#ifdef _OPENMP
  omp_set_num_threads(n > 0 ? n : 1);
#else
  (void)n;
#endif
}
int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
int orc_hw_threads(void) { return (int)std::thread::hardware_concurrency(); }

// Decoders of whole arrays (kind 0 bf16, 1 binary16, 2 E2M1 codes as bytes,
// 3 E8M0, 4 E4M3) and the two rounding conversions.
void orc_decode(int kind, const void* in, long long n, double* out) {
  for (long long i = 0; i < n; ++i) {
    if (kind == 0) out[i] = orc::bf16_to_f64(static_cast<const uint16_t*>(in)[i]);
    else if (kind == 1) out[i] = orc::f16_to_f64(static_cast<const uint16_t*>(in)[i]);
    else if (kind == 2) out[i] = orc::e2m1_to_f64(static_cast<const uint8_t*>(in)[i]);
    else if (kind == 3) out[i] = orc::e8m0_to_f64(static_cast<const uint8_t*>(in)[i]);
    else out[i] = orc::e4m3_to_f64(static_cast<const uint8_t*>(in)[i]);
  }
}
void orc_to_bf16(const double* x, long long n, uint16_t* out) {
  for (long long i = 0; i < n; ++i) out[i] = orc::f64_to_bf16(x[i]);
}
void orc_to_f16(const double* x, long long n, uint16_t* out) {
  for (long long i = 0; i < n; ++i) out[i] = orc::f64_to_f16(x[i]);
}

// Stored rows [rows][K/2] -> codes [rows][K] in element order.
void orc_unpack_codes(const uint8_t* q, long long rows, int K, uint8_t* u) {
  for (long long r = 0; r < rows; ++r)
    for (int k = 0; k < K; ++k) u[r * K + k] = (uint8_t)orc::code_at(q + r * (K / 2), k);
}

// Codes [rows][K] (0..15) -> stored rows [rows][K/2].
void orc_pack_codes(const uint8_t* u, long long rows, int K, uint8_t* q) {
  for (long long r = 0; r < rows; ++r) {
    uint8_t* row = q + r * (K / 2);
    for (int b = 0; b < K / 2; ++b) row[b] = 0;
    for (int k = 0; k < K; ++k) {
      const int t = k / 128, j = (k % 128) / 32, qq = (k % 32) / 8, e = k % 8;
      row[64 * t + 16 * qq + 4 * j + e / 2] |= (uint8_t)((u[r * K + k] & 0xF) << (4 * (e & 1)));
    }
  }
}

// Stored matrix (rows x K, format fmt, matrix scale ts for NVFP4) -> fp64.
void orc_dequant(const uint8_t* q, const void* s, float ts, int fmt, long long rows, int K, double* w) {
  const orc_mat m{q, s, &ts};
  for (long long r = 0; r < rows; ++r) {
    orc_mat mr = m;
    dequant_row(mr, fmt, 0, (size_t)rows, K, (size_t)r, w + r * K);
  }
}

// The int4 quantizer (offline; produces stored weights): per group of 32,
// a = max|w|, s = binary16(a / 7) (fp64 quotient, rounded to nearest even);
// s == 0 gives codes 8, else q = clamp(round_half_even(w / s), -7, 7), u = q + 8.
void orc_quantize_int4(const float* w, long long rows, int K, uint8_t* u, uint16_t* sbits) {
  for (long long r = 0; r < rows; ++r)
    for (int g = 0; g < K / 32; ++g) {
      const float* wg = w + r * K + 32 * g;
      double a = 0.0;
      for (int i = 0; i < 32; ++i) a = std::max(a, std::fabs((double)wg[i]));
      const uint16_t sb = orc::f64_to_f16(a / 7.0);
      sbits[r * (K / 32) + g] = sb;
      const double s = orc::f16_to_f64(sb);
      for (int i = 0; i < 32; ++i) {
        double q = 0.0;
        if (s != 0.0) q = std::min(7.0, std::max(-7.0, std::nearbyint((double)wg[i] / s)));
        u[r * K + 32 * g + i] = (uint8_t)(q + 8.0);
      }
    }
}

// Router logits of one bf16 token.
void orc_router(const orc_layer* L, const uint16_t* x_bits, double* logits) {
  std::vector<double> x(L->d);
  to_f64(x_bits, L->d, x.data());
  router(L, x.data(), logits);
}

// Chosen set S (k largest logits, larger first, lower index on ties) and its
// weights w from E logits.
void orc_route(const double* l, int E, int k, int norm, int32_t* S, double* w) {
  std::vector<int> order(E);
  for (int e = 0; e < E; ++e) order[e] = e;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return l[a] > l[b]; });
  double mx = l[0];
  for (int e = 1; e < E; ++e) mx = std::max(mx, l[e]);
  std::vector<double> p(E);
  double z = 0.0;
  for (int e = 0; e < E; ++e) {
    p[e] = std::exp(l[e] - mx);
    z += p[e];
  }
  for (int e = 0; e < E; ++e) p[e] /= z;
  double ps = 0.0;
  for (int j = 0; j < k; ++j) {
    S[j] = order[j];
    ps += p[order[j]];
  }
  for (int j = 0; j < k; ++j) w[j] = norm ? p[S[j]] / ps : p[S[j]];
}

// One token through one layer with the chosen set S (n experts, their
// weights w) given; y [d] in fp64.  Adds the weights read to *read.
static void layer_on_set(const orc_layer* L, const double* x, const int32_t* S, const double* w, int n, double* y,
                         long long* read) {
  const int d = L->d, f = L->f;
  std::vector<int> asc(n);
  for (int j = 0; j < n; ++j) asc[j] = j;
  std::stable_sort(asc.begin(), asc.end(), [&](int a, int b) { return S[a] < S[b]; });
  std::vector<double> o(d);
  for (int i = 0; i < d; ++i) y[i] = 0.0;
  for (int jj = 0; jj < n; ++jj) {
    const int j = asc[jj];
    expert_forward(L, L->gate, L->up, L->down, (size_t)S[j], x, o.data());
    for (int i = 0; i < d; ++i) y[i] += w[j] * o[i];
  }
  *read += (long long)n * 3 * d * f;
  if (L->has_shared) {
    expert_forward(L, L->sh_gate, L->sh_up, L->sh_down, 0, x, o.data());
    for (int i = 0; i < d; ++i) y[i] += o[i];
    *read += 3LL * d * f;
  }
}

// One bf16 token through one layer: only the chosen experts are evaluated.
// Outputs y [d] (fp64), idx [k], w [k], logits [E]; *read (if not NULL)
// receives the number of weights read (router E d plus 3 d f per expert run).
void orc_moe_forward(const orc_layer* L, const uint16_t* x_bits, int k, int norm, double* y, int32_t* idx,
                     double* w, double* logits, long long* read) {
  std::vector<double> x(L->d);
  to_f64(x_bits, L->d, x.data());
  router(L, x.data(), logits);
  long long rd = (long long)L->E * L->d;
  orc_route(logits, L->E, k, norm, idx, w);
  layer_on_set(L, x.data(), idx, w, k, y, &rd);
  if (read) *read = rd;
}

// The same token with the chosen set S (n experts) given instead of selected:
// weights are the softmax over all E restricted to S, renormalized over S
// when norm.
void orc_moe_forward_on_set(const orc_layer* L, const uint16_t* x_bits, const int32_t* S, int n, int norm,
                            double* y, double* w) {
  const int E = L->E;
  std::vector<double> x(L->d), l(E), p(E);
  to_f64(x_bits, L->d, x.data());
  router(L, x.data(), l.data());
  double mx = l[0];
  for (int e = 1; e < E; ++e) mx = std::max(mx, l[e]);
  double z = 0.0;
  for (int e = 0; e < E; ++e) {
    p[e] = std::exp(l[e] - mx);
    z += p[e];
  }
  double ps = 0.0;
  for (int j = 0; j < n; ++j) ps += p[S[j]] / z;
  for (int j = 0; j < n; ++j) w[j] = norm ? (p[S[j]] / z) / ps : p[S[j]] / z;
  long long rd = 0;
  layer_on_set(L, x.data(), S, w, n, y, &rd);
}

// Brute force: every expert evaluated, then kept by a 0/1 mask times its
// weight, y = sum_{e=0}^{E-1} (m_e w_e) o_e in ascending e (plus the shared
// expert with mask 1).
void orc_moe_forward_masked(const orc_layer* L, const uint16_t* x_bits, int k, int norm, double* y,
                            long long* read) {
  const int d = L->d, f = L->f, E = L->E;
  std::vector<double> x(d), l(E), w(k), mw(E, 0.0), o(d);
  std::vector<int32_t> S(k);
  to_f64(x_bits, d, x.data());
  router(L, x.data(), l.data());
  orc_route(l.data(), E, k, norm, S.data(), w.data());
  for (int j = 0; j < k; ++j) mw[S[j]] = w[j];
  for (int i = 0; i < d; ++i) y[i] = 0.0;
  for (int e = 0; e < E; ++e) {
    expert_forward(L, L->gate, L->up, L->down, (size_t)e, x.data(), o.data());
    for (int i = 0; i < d; ++i) y[i] += mw[e] * o[i];
  }
  long long rd = (long long)E * d + (long long)E * 3 * d * f;
  if (L->has_shared) {
    expert_forward(L, L->sh_gate, L->sh_up, L->sh_down, 0, x.data(), o.data());
    for (int i = 0; i < d; ++i) y[i] += 1.0 * o[i];
    rd += 3LL * d * f;
  }
  if (read) *read = rd;
}

// x = bf16(r / sqrt(mean(r^2) + eps)), unit weight.
void orc_rmsnorm_bf16(const float* r, int d, double eps, uint16_t* x) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += (double)r[i] * (double)r[i];
  const double den = std::sqrt(ss / d + eps);
  for (int i = 0; i < d; ++i) x[i] = orc::f64_to_bf16((double)r[i] / den);
}

// The pre-norm stack of nl layers for one token x0 (bf16): r (fp32, [d]) is
// the residual after the last layer; xs [nl][d] (bf16 bits), ys [nl][d]
// (fp32) and idx [nl][k] record every layer (each may be NULL).
void orc_stack_forward(const orc_layer* const* layers, int nl, const uint16_t* x0, int k, double eps, int norm,
                       float* r, uint16_t* xs, float* ys, int32_t* idx) {
  const int d = layers[0]->d;
  std::vector<uint16_t> x(d);
  std::vector<double> y(d), w(k), lg;
  std::vector<int32_t> S(k);
  for (int i = 0; i < d; ++i) r[i] = (float)orc::bf16_to_f64(x0[i]);
  for (int l = 0; l < nl; ++l) {
    const orc_layer* L = layers[l];
    orc_rmsnorm_bf16(r, d, eps, x.data());
    lg.assign(L->E, 0.0);
    orc_moe_forward(L, x.data(), k, norm, y.data(), S.data(), w.data(), lg.data(), nullptr);
    for (int i = 0; i < d; ++i) {
      const float y32 = (float)y[i];
      if (ys) ys[(size_t)l * d + i] = y32;
      if (xs) xs[(size_t)l * d + i] = x[i];
      r[i] = (float)((double)r[i] + (double)y32);
    }
    if (idx)
      for (int j = 0; j < k; ++j) idx[(size_t)l * k + j] = S[j];
  }
}

// The T*k assignments a = t*k + j (token t's j-th expert idx[a]) grouped by
// expert: off [E+1] (expert e owns positions off[e] .. off[e+1]-1), order
// [T*k] (ascending a within an expert), active [E] (experts owning any,
// ascending; *n_active of them).
void orc_group_by_expert(const int32_t* idx, int Tk, int E, int32_t* off, int32_t* order, int32_t* active,
                         int32_t* n_active) {
  int p = 0, na = 0;
  for (int e = 0; e < E; ++e) {
    off[e] = p;
    for (int a = 0; a < Tk; ++a)
      if (idx[a] == e) order[p++] = a;
    if (p > off[e]) active[na++] = e;
  }
  off[E] = p;
  *n_active = na;
}

}  // extern "C"
