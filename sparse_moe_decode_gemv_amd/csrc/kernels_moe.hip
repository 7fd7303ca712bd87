// kernels_moe.hip -- one decode step of a 4-bit MoE layer on gfx950.
//
// Three kernels per call, each HBM-streaming and wave64-native:
//   router  : logits = W_r x (+b), fp32 weights, one router row per wave;
//             the last workgroup to finish a token (arrival counter) does the
//             softmax and top-k of that token in one wave.  In the stack the
//             router also applies the pre-norm (RMSNorm) to the residual.
//   gateup  : for the chosen experts only, g = W_g x and u = W_u x from int4
//             pieces (one 16-byte piece per lane per load, x held in
//             registers), h = w_j * silu(g) * u.
//   down    : y = sum_j W_d[j] h_j; each output row is reduced inside one
//             wave (no atomics, deterministic); in the stack the residual
//             add is folded in.
// The pages describe the step these kernels compute: per token a small
// router selects a few of 256 routed experts and only those run ("Flint 40B:
// Best Mid Sized LLM", transcript 02:35); dedicated kernels for low-bit
// projections and MoE routing are named in the same source (06:11).
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"
#include "topk.h"

namespace moe {

// ----------------------------------------------------------------- top-k

// Softmax + top-k of one token's E logits in one wave (topk.h); lane r < k
// writes choice r.
template <int EPL>
__device__ __forceinline__ void topk_wave(const float* lg, int E, int k, int norm, int lane, int32_t* sel_idx,
                                          float* sel_w, int32_t* idx_out, float* w_out) {
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const float l = load_coherent(lg + min(lane + 64 * i, E - 1));
    v[i] = lane + 64 * i < E && l == l ? l : -INFINITY;
  }
  int se;
  float sw;
  topk_fast<EPL>(v, E, k, norm, lane, se, sw);
  if (lane < k) {
    sel_idx[lane] = se;
    sel_w[lane] = sw;
    if (idx_out) idx_out[lane] = se;
    if (w_out) w_out[lane] = sw;
  }
}

// ----------------------------------------------------------------- router

// grid (E, T), block 64: wave e of token t computes logit e.  EPL = experts
// per lane in the top-k wave, ceil(E/64).
template <int D, int EPL>
__global__ __launch_bounds__(64) void k_router(const float* __restrict__ Wr, const float* __restrict__ bias,
                                               const uint16_t* __restrict__ x, const float* __restrict__ resid,
                                               float eps, int E, int k, int norm, float* __restrict__ logits,
                                               unsigned* __restrict__ counters, int32_t* __restrict__ sel_idx,
                                               float* __restrict__ sel_w, int32_t* __restrict__ idx_out,
                                               float* __restrict__ w_out, uint16_t* __restrict__ xnorm,
                                               uint16_t* __restrict__ x_trace) {
  constexpr int NI = D / 256;  // float4 columns per lane: 4*lane + 256*i
  const int e = blockIdx.x, t = blockIdx.y, lane = threadIdx.x;
  const float4* wrow = reinterpret_cast<const float4*>(Wr + (size_t)e * D);
  float4 w[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) w[i] = wrow[64 * i + lane];

  float xv[NI][4];
  if (x) {
    const uint2* xr = reinterpret_cast<const uint2*>(x + (size_t)t * D);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint2 q = xr[64 * i + lane];
      xv[i][0] = bf16_bits_to_f32(q.x & 0xFFFFu);
      xv[i][1] = bf16_bits_to_f32(q.x >> 16);
      xv[i][2] = bf16_bits_to_f32(q.y & 0xFFFFu);
      xv[i][3] = bf16_bits_to_f32(q.y >> 16);
    }
  } else {
    // pre-norm: x = bf16(r / sqrt(mean(r^2) + eps))
    const float4* rr = reinterpret_cast<const float4*>(resid + (size_t)t * D);
    float4 rv[NI];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      rv[i] = rr[64 * i + lane];
      ss = fmaf(rv[i].x, rv[i].x, ss);
      ss = fmaf(rv[i].y, rv[i].y, ss);
      ss = fmaf(rv[i].z, rv[i].z, ss);
      ss = fmaf(rv[i].w, rv[i].w, ss);
    }
    ss = wave_sum(ss);
    const float den = sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t b0 = f32_to_bf16_bits(rv[i].x / den), b1 = f32_to_bf16_bits(rv[i].y / den);
      const uint32_t b2 = f32_to_bf16_bits(rv[i].z / den), b3 = f32_to_bf16_bits(rv[i].w / den);
      xv[i][0] = bf16_bits_to_f32(b0);
      xv[i][1] = bf16_bits_to_f32(b1);
      xv[i][2] = bf16_bits_to_f32(b2);
      xv[i][3] = bf16_bits_to_f32(b3);
      if (e == 0) {
        const uint2 pk = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        reinterpret_cast<uint2*>(xnorm + (size_t)t * D)[64 * i + lane] = pk;
        if (x_trace) reinterpret_cast<uint2*>(x_trace + (size_t)t * D)[64 * i + lane] = pk;
      }
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    acc = fmaf(w[i].x, xv[i][0], acc);
    acc = fmaf(w[i].y, xv[i][1], acc);
    acc = fmaf(w[i].z, xv[i][2], acc);
    acc = fmaf(w[i].w, xv[i][3], acc);
  }
  acc = wave_sum(acc);
  if (bias) acc += bias[e];
  if (lane == 0) store_coherent(logits + (size_t)t * E + e, acc);

  // Arrival: the last wave of token t selects its experts.
  wait_vm();
  unsigned prev = 0;
  if (lane == 0) prev = arrive(&counters[t]);
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev != (unsigned)(E - 1)) return;
  const float* lg = logits + (size_t)t * E;
  int32_t* io = idx_out ? idx_out + (size_t)t * k : nullptr;
  float* wo = w_out ? w_out + (size_t)t * k : nullptr;
  topk_wave<EPL>(lg, E, k, norm, lane, sel_idx + t * k, sel_w + t * k, io, wo);
  if (lane == 0) counters[t] = 0u;  // ready for the next call
}

// ----------------------------------------------------------------- gate/up

// A wave covers 64*NL consecutive 16-byte pieces of the gate matrix of one
// chosen expert (and the same pieces of its up matrix).  CPR = pieces per
// row = d/32.
template <int CPR, int NL>
__global__ __launch_bounds__(256) void k_gateup(const uint16_t* __restrict__ x, const uint8_t* __restrict__ gq,
                                                const uint16_t* __restrict__ gs, const uint8_t* __restrict__ uq,
                                                const uint16_t* __restrict__ us,
                                                const int32_t* __restrict__ sel_idx,
                                                const float* __restrict__ sel_w, int f, int k, int E,
                                                float* __restrict__ h) {
  constexpr int D = CPR * 32;
  constexpr int XS = CPR > 64 ? CPR / 64 : 1;
  constexpr int LPR = CPR > 64 ? CPR / 64 : 1;
  static_assert(NL % LPR == 0, "a wave must cover whole rows");
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = blockIdx.y;
  const int waves_per_expert = (f * CPR) / (64 * NL);
  const int slot = wave / waves_per_expert;
  if (slot >= k) return;
  const int c0 = (wave - slot * waves_per_expert) * 64 * NL;
  const int e = min(max(sel_idx[t * k + slot], 0), E - 1);  // never read outside the expert arrays
  const float wj = sel_w[t * k + slot];
  const size_t mat_pieces = (size_t)f * CPR;
  const uint4* gp = reinterpret_cast<const uint4*>(gq) + (size_t)e * mat_pieces;
  const uint4* up = reinterpret_cast<const uint4*>(uq) + (size_t)e * mat_pieces;
  const uint16_t* gsb = gs + (size_t)e * mat_pieces;  // CPR scales per row
  const uint16_t* usb = us + (size_t)e * mat_pieces;

  uint4 qg[NL], qu[NL];
  uint2 sg[NL], su[NL];
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int c = c0 + 64 * n + lane;
    qg[n] = gp[c];
    qu[n] = up[c];
    const int row = c / CPR, cc = c % CPR;
    const size_t so = (size_t)row * CPR + (cc & ~3);
    sg[n] = *reinterpret_cast<const uint2*>(gsb + so);
    su[n] = *reinterpret_cast<const uint2*>(usb + so);
  }

  Slice8 xs[XS][4];
  const uint4* xp = reinterpret_cast<const uint4*>(x + (size_t)t * D);
#pragma unroll
  for (int s = 0; s < XS; ++s) {
    const int cc = CPR > 64 ? 64 * s + lane : lane % CPR;
    const int base = 128 * (cc >> 2) + 8 * (cc & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) xs[s][j] = make_slice_bf16(xp[(base + 32 * j) >> 3]);
  }

  float* hout = h + ((size_t)t * k + slot) * f;
  float ag = 0.f, au = 0.f;
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int s = CPR > 64 ? n % XS : 0;
    ag += dot_piece(qg[n], xs[s], sg[n]);
    au += dot_piece(qu[n], xs[s], su[n]);
    if (n % LPR == LPR - 1) {
      if constexpr (CPR >= 64) {
        const float g = wave_sum(ag), u = wave_sum(au);
        if (lane == 0) hout[(c0 + 64 * n) / CPR] = wj * silu(g) * u;
      } else {
        const float g = seg_sum<CPR>(ag), u = seg_sum<CPR>(au);
        if (lane % CPR == 0) hout[(c0 + 64 * n + lane) / CPR] = wj * silu(g) * u;
      }
      ag = au = 0.f;
    }
  }
}

// ----------------------------------------------------------------- down

// Output row r needs P = KP*CPRF pieces (KP = top_k rounded up to a power of
// two, CPRF = f/32 pieces per expert row).  Lane l always handles the same
// (slot, piece) pairs, so its activation slices stay in registers.
template <int CPRF, int KP>
__global__ __launch_bounds__(256) void k_down(const float* __restrict__ h, const uint8_t* __restrict__ dq,
                                              const uint16_t* __restrict__ ds,
                                              const int32_t* __restrict__ sel_idx, int d, int k, int E,
                                              float* __restrict__ y_out, float* __restrict__ resid) {
  constexpr int F = CPRF * 32;
  constexpr int P = KP * CPRF;
  constexpr int LPR = P > 64 ? P / 64 : 1;
  constexpr int RPL = P < 64 ? 64 / P : 1;
  constexpr int NLD = LPR > 4 ? LPR : 4;
  constexpr int ROWS_W = (NLD / LPR) * RPL;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = blockIdx.y;
  const int r0 = wave * ROWS_W;
  if (r0 >= d) return;

  int cc[LPR], slot[LPR];
  bool act[LPR];
  size_t ebase[LPR];
#pragma unroll
  for (int m = 0; m < LPR; ++m) {
    const int flat = P >= 64 ? 64 * m + lane : lane % P;
    slot[m] = flat / CPRF;
    cc[m] = flat % CPRF;
    act[m] = slot[m] < k;
    const int e = act[m] ? min(max(sel_idx[t * k + slot[m]], 0), E - 1) : 0;
    ebase[m] = (size_t)e * d;
  }

  // weight pieces first: their HBM latency overlaps the activation set-up
  uint4 q[NLD];
  uint2 sc[NLD];
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    const int m = n % LPR;
    const int row = r0 + (P >= 64 ? n / LPR : n * RPL + lane / P);
    if (act[m]) {
      q[n] = *reinterpret_cast<const uint4*>(dq + piece_offset(ebase[m] + row, CPRF, cc[m]));
      sc[n] = *reinterpret_cast<const uint2*>(ds + (ebase[m] + row) * CPRF + (cc[m] & ~3));
    } else {
      q[n] = make_uint4(0, 0, 0, 0);
      sc[n] = make_uint2(0, 0);
    }
  }

  Slice8 hs8[LPR][4];
#pragma unroll
  for (int m = 0; m < LPR; ++m) {
    const int base = 128 * (cc[m] >> 2) + 8 * (cc[m] & 3);
    const float* hs = h + ((size_t)t * k + (act[m] ? slot[m] : 0)) * F;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[8];
      const float4 a = *reinterpret_cast<const float4*>(hs + base + 32 * j);
      const float4 b = *reinterpret_cast<const float4*>(hs + base + 32 * j + 4);
      const bool on = act[m];  // padding slots contribute exact zeros
      v[0] = on ? a.x : 0.f, v[1] = on ? a.y : 0.f, v[2] = on ? a.z : 0.f, v[3] = on ? a.w : 0.f;
      v[4] = on ? b.x : 0.f, v[5] = on ? b.y : 0.f, v[6] = on ? b.z : 0.f, v[7] = on ? b.w : 0.f;
      hs8[m][j] = make_slice_f16(v);
    }
  }

  float acc = 0.f;
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    const int m = n % LPR;
    acc += dot_piece_f16(q[n], hs8[m], sc[n]);
    if (n % LPR == LPR - 1) {
      float v;
      int row;
      bool writer;
      if constexpr (P >= 64) {
        v = wave_sum(acc);
        row = r0 + n / LPR;
        writer = lane == 0;
      } else {
        v = seg_sum<P>(acc);
        row = r0 + n * RPL + lane / P;
        writer = lane % P == 0;
      }
      if (writer) {
        const size_t o = (size_t)t * d + row;
        if (resid) resid[o] += v;
        if (y_out) y_out[o] = v;
      }
      acc = 0.f;
    }
  }
}

// ----------------------------------------------------------------- launchers

template <int D, int EPL>
static void router_launch(const LayerArgs& a, const uint16_t* x, const float* r, float eps, int T, int32_t* io,
                          float* wo, uint16_t* xt, hipStream_t s) {
  hipLaunchKernelGGL((k_router<D, EPL>), dim3(a.E, T), dim3(64), 0, s, a.router_w, a.router_b, x, r, eps, a.E,
                     a.k, a.norm_topk, a.logits, a.counters, a.sel_idx, a.sel_w, io, wo, a.xnorm, xt);
}

template <int D>
static void router_inst(const LayerArgs& a, const uint16_t* x, const float* r, float eps, int T, int32_t* io,
                        float* wo, uint16_t* xt, hipStream_t s) {
  const int epl = (a.E + 63) / 64;
  if (epl <= 1)
    router_launch<D, 1>(a, x, r, eps, T, io, wo, xt, s);
  else if (epl <= 2)
    router_launch<D, 2>(a, x, r, eps, T, io, wo, xt, s);
  else if (epl <= 4)
    router_launch<D, 4>(a, x, r, eps, T, io, wo, xt, s);
  else if (epl <= 8)
    router_launch<D, 8>(a, x, r, eps, T, io, wo, xt, s);
  else
    router_launch<D, 16>(a, x, r, eps, T, io, wo, xt, s);
}

hipError_t launch_router(const LayerArgs& a, const uint16_t* x, const float* r, float eps, int T,
                         int32_t* idx_out, float* w_out, uint16_t* x_trace, hipStream_t s) {
  switch (a.d) {
    case 256: router_inst<256>(a, x, r, eps, T, idx_out, w_out, x_trace, s); break;
    case 512: router_inst<512>(a, x, r, eps, T, idx_out, w_out, x_trace, s); break;
    case 1024: router_inst<1024>(a, x, r, eps, T, idx_out, w_out, x_trace, s); break;
    case 2048: router_inst<2048>(a, x, r, eps, T, idx_out, w_out, x_trace, s); break;
    case 4096: router_inst<4096>(a, x, r, eps, T, idx_out, w_out, x_trace, s); break;
    case 8192: router_inst<8192>(a, x, r, eps, T, idx_out, w_out, x_trace, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int CPR>
static void gateup_inst(const LayerArgs& a, const uint16_t* x, int T, hipStream_t s) {
  constexpr int NL = 4;
  const int waves = a.k * (a.f * CPR) / (64 * NL);
  hipLaunchKernelGGL((k_gateup<CPR, NL>), dim3((waves + 3) / 4, T), dim3(256), 0, s, x, a.gate_q, a.gate_s,
                     a.up_q, a.up_s, a.sel_idx, a.sel_w, a.f, a.k, a.E, a.h);
}

hipError_t launch_gateup(const LayerArgs& a, const uint16_t* x, int T, hipStream_t s) {
  switch (a.d / 32) {
    case 8: gateup_inst<8>(a, x, T, s); break;
    case 16: gateup_inst<16>(a, x, T, s); break;
    case 32: gateup_inst<32>(a, x, T, s); break;
    case 64: gateup_inst<64>(a, x, T, s); break;
    case 128: gateup_inst<128>(a, x, T, s); break;
    case 256: gateup_inst<256>(a, x, T, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int CPRF, int KP>
static void down_inst(const LayerArgs& a, int T, float* y, float* resid, hipStream_t s) {
  constexpr int P = KP * CPRF;
  constexpr int LPR = P > 64 ? P / 64 : 1;
  constexpr int RPL = P < 64 ? 64 / P : 1;
  constexpr int NLD = LPR > 4 ? LPR : 4;
  constexpr int ROWS_W = (NLD / LPR) * RPL;
  const int waves = a.d / ROWS_W;
  hipLaunchKernelGGL((k_down<CPRF, KP>), dim3((waves + 3) / 4, T), dim3(256), 0, s, a.h, a.down_q, a.down_s,
                     a.sel_idx, a.d, a.k, a.E, y, resid);
}

template <int CPRF>
static hipError_t down_kp(const LayerArgs& a, int T, float* y, float* resid, hipStream_t s) {
  const int kp = a.k <= 1 ? 1 : a.k <= 2 ? 2 : a.k <= 4 ? 4 : a.k <= 8 ? 8 : 16;
  switch (kp) {
    case 1: down_inst<CPRF, 1>(a, T, y, resid, s); break;
    case 2: down_inst<CPRF, 2>(a, T, y, resid, s); break;
    case 4: down_inst<CPRF, 4>(a, T, y, resid, s); break;
    case 8: down_inst<CPRF, 8>(a, T, y, resid, s); break;
    default: down_inst<CPRF, 16>(a, T, y, resid, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_down(const LayerArgs& a, int T, float* y_out, float* residual, hipStream_t s) {
  switch (a.f / 32) {
    case 4: return down_kp<4>(a, T, y_out, residual, s);
    case 8: return down_kp<8>(a, T, y_out, residual, s);
    case 16: return down_kp<16>(a, T, y_out, residual, s);
    case 32: return down_kp<32>(a, T, y_out, residual, s);
    case 64: return down_kp<64>(a, T, y_out, residual, s);
    case 128: return down_kp<128>(a, T, y_out, residual, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
