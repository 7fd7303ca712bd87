// kernels_layer.hip -- the whole 1-token MoE layer step in one launch (gfx950).
//
// Per token a small router picks a few of 256 routed experts and only those
// run ("Flint 40B: Best Mid Sized LLM", transcript 02:35).  The step is a
// chain of dependent phases -- router GEMV, top-k, expert gate/up + SwiGLU,
// down + combine -- and at one token each phase moves only a few MB, so the
// cost is latency, not bandwidth.  On MI355X a kernel boundary in a graph
// costs about 1.6 us and a counter-based grid barrier over 256 workgroups
// about 3.7 us (same-address atomics serialize), so this kernel keeps every
// workgroup resident (grid = one workgroup per CU) and passes data between
// phases without atomics:
//
//   router   each workgroup computes one router row (its 4 waves take a
//            quarter each) and publishes the logit as a 64-bit word
//            (epoch << 32 | value) with a coherent store;
//   select   wave 0 of every workgroup polls the E tagged words until all
//            carry this call's epoch, then runs the exact top-k itself (no
//            second hand-off);
//   experts  each wave issues its down-projection loads at once (the chosen
//            experts are known now), then its gate/up rows; h = w_j *
//            silu(g) * u goes out with coherent stores and the workgroup
//            raises its flag (= epoch);
//   down     wave 0 polls the G flags, the workgroup copies h into LDS, and
//            each wave finishes its output rows from the prefetched weights.
//
// The epoch is read from the workspace at the start and advanced by
// workgroup 0 once every flag is up (by then every workgroup has read it),
// so consecutive calls never see each other's tags.  Every wait is bounded:
// on timeout the kernel sets the error word and finishes anyway.
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"
#include "topk.h"

namespace moe {

constexpr unsigned kSpinLimit = 1u << 21;

__device__ __forceinline__ void store_tagged(unsigned long long* p, float v, unsigned tag) {
  store_coherent(p, ((unsigned long long)tag << 32) | (unsigned long long)__float_as_uint(v));
}
__device__ __forceinline__ void store_coherent_u32(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned load_coherent_u32(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every poll below issues all of its coherent loads before looking at any
// result, so one poll costs one round trip to the coherence point (about
// 0.6 us on MI355X), not one per load.

// Wave-wide: wait until the E tagged logits carry `tag`; v receives them
// (NaN mapped to -inf, entries past E to -inf).
template <int EPL>
__device__ void poll_logits(const unsigned long long* lg, int E, unsigned tag, int lane, float v[EPL],
                            unsigned* error) {
  for (unsigned spin = 0;; ++spin) {
    unsigned long long t[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) t[i] = load_coherent(lg + min(lane + 64 * i, E - 1));
    bool ok = true;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const bool valid = lane + 64 * i < E;
      const float f = __uint_as_float((uint32_t)t[i]);
      v[i] = valid && f == f ? f : -INFINITY;
      ok = ok & (!valid | ((uint32_t)(t[i] >> 32) == tag));
    }
    if (__builtin_amdgcn_ballot_w64(!ok) == 0) return;
    if (spin > kSpinLimit) {
      if (lane == 0) atomicOr(error, 1u);
      return;
    }
  }
}

// Wave-wide: wait until flags[0..G) all equal `tag` (G even, <= 1024).
__device__ void poll_flags(const unsigned* flags, int G, unsigned tag, int lane, unsigned* error) {
  const unsigned long long* f2 = reinterpret_cast<const unsigned long long*>(flags);
  const unsigned long long want = ((unsigned long long)tag << 32) | tag;
  const int pairs = G / 2;
  for (unsigned spin = 0;; ++spin) {
    unsigned long long f[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) f[m] = load_coherent(f2 + min(lane + 64 * m, pairs - 1));
    bool ok = true;
#pragma unroll
    for (int m = 0; m < 8; ++m) ok = ok & (f[m] == want);
    if (__builtin_amdgcn_ballot_w64(!ok) == 0) return;
    if (spin > kSpinLimit) {
      if (lane == 0) atomicOr(error, 2u);
      return;
    }
  }
}

// D hidden, F expert width, KP top_k rounded up to a power of two, EPL
// experts per lane in the top-k wave, RW waves per router row.
template <int D, int F, int KP, int EPL, int RW>
__global__ __launch_bounds__(256) void k_layer(FusedArgs a) {
  constexpr int CPR = D / 32;        // 16-byte pieces per gate/up row
  constexpr int CPRF = F / 32;       // pieces per down row
  constexpr int NL = 4;              // gate (and up) loads per lane
  constexpr int XS = CPR > 64 ? CPR / 64 : 1;
  constexpr int LPRG = CPR > 64 ? CPR / 64 : 1;
  constexpr int P = KP * CPRF;       // pieces per output row
  constexpr int LPRD = P > 64 ? P / 64 : 1;
  constexpr int RPLD = P < 64 ? 64 / P : 1;
  constexpr int NLD = LPRD > 4 ? LPRD : 4;
  constexpr int ROWS_W = (NLD / LPRD) * RPLD;
  constexpr int NI = D / (RW * 256);  // router float4 per lane
  static_assert(NL % LPRG == 0 && NI >= 1, "shape");

  extern __shared__ float s_h[];      // k * F
  __shared__ int s_idx[16];
  __shared__ float s_w[16];
  __shared__ float s_part[4];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int G = gridDim.x, W = 4 * G, wg = blockIdx.x * 4 + wid;
  const int E = a.E, k = a.k;
  const unsigned tag = load_coherent_u32(a.epoch) + 1u;

  // ---------------------------------------------------------------- router
  {
    const int row = wg / RW, part = wg % RW;
    if (row < E) {
      const float4* wr = reinterpret_cast<const float4*>(a.router_w + (size_t)row * D + part * (D / RW));
      const uint2* xr = reinterpret_cast<const uint2*>(a.x + part * (D / RW));
      float4 w[NI];
      uint2 q[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) w[i] = wr[64 * i + lane], q[i] = xr[64 * i + lane];
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        acc = fmaf(w[i].x, bf16_bits_to_f32(q[i].x & 0xFFFFu), acc);
        acc = fmaf(w[i].y, __uint_as_float(q[i].x & 0xFFFF0000u), acc);
        acc = fmaf(w[i].z, bf16_bits_to_f32(q[i].y & 0xFFFFu), acc);
        acc = fmaf(w[i].w, __uint_as_float(q[i].y & 0xFFFF0000u), acc);
      }
      acc = wave_sum(acc);
      if (RW == 1) {
        if (lane == 0) store_tagged(a.logits + row, acc + (a.router_b ? a.router_b[row] : 0.f), tag);
      } else if (lane == 0) {
        s_part[wid] = acc;
      }
    }
    if (RW > 1) {
      __syncthreads();
      if (threadIdx.x < 4 / RW) {
        const int r = (blockIdx.x * 4) / RW + threadIdx.x;
        if (r < E) {
          float sum = 0.f;
#pragma unroll
          for (int p = 0; p < RW; ++p) sum += s_part[threadIdx.x * RW + p];
          store_tagged(a.logits + r, sum + (a.router_b ? a.router_b[r] : 0.f), tag);
        }
      }
    }
  }

  // ---------------------------------------------------------------- select
  if (wid == 0) {
    float v[EPL];
    poll_logits<EPL>(a.logits, E, tag, lane, v, a.error);
    int se;
    float sw;
    topk_fast<EPL>(v, E, k, a.norm, lane, se, sw);
    if (lane < k) {
      s_idx[lane] = se;
      s_w[lane] = sw;
      if (blockIdx.x == 0) {
        if (a.idx_out) a.idx_out[lane] = se;
        if (a.w_out) a.w_out[lane] = sw;
      }
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- down prefetch
  const bool has_down = wg < D / ROWS_W;
  const int r0 = wg * ROWS_W;
  int cc[LPRD], dslot[LPRD];
  bool act[LPRD];
  uint4 qd[NLD];
  uint2 sd[NLD];
#pragma unroll
  for (int m = 0; m < LPRD; ++m) {
    const int flat = P >= 64 ? 64 * m + lane : lane % P;
    dslot[m] = flat / CPRF;
    cc[m] = flat % CPRF;
    act[m] = has_down && dslot[m] < k;
  }
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    const int m = n % LPRD;
    const int row = r0 + (P >= 64 ? n / LPRD : n * RPLD + lane / P);
    if (act[m]) {
      const size_t eb = (size_t)min(max(s_idx[dslot[m]], 0), E - 1) * D + row;
      qd[n] = *reinterpret_cast<const uint4*>(a.down_q + piece_offset(eb, CPRF, cc[m]));
      sd[n] = *reinterpret_cast<const uint2*>(a.down_s + eb * CPRF + (cc[m] & ~3));
    } else {
      qd[n] = make_uint4(0, 0, 0, 0);
      sd[n] = make_uint2(0, 0);
    }
  }

  // ---------------------------------------------------------------- gate/up
  {
    const int wpe = (F * CPR) / (64 * NL);  // waves per chosen expert
    if (wg < k * wpe) {
      const int slot = wg / wpe;
      const int c0 = (wg - slot * wpe) * 64 * NL;
      const int e = min(max(s_idx[slot], 0), E - 1);
      const float wj = s_w[slot];
      const size_t mat = (size_t)F * CPR;
      const uint4* gp = reinterpret_cast<const uint4*>(a.gate_q) + (size_t)e * mat;
      const uint4* up = reinterpret_cast<const uint4*>(a.up_q) + (size_t)e * mat;
      const uint16_t* gsb = a.gate_s + (size_t)e * mat;
      const uint16_t* usb = a.up_s + (size_t)e * mat;
      uint4 qg[NL], qu[NL];
      uint2 sg[NL], su[NL];
#pragma unroll
      for (int n = 0; n < NL; ++n) {
        const int c = c0 + 64 * n + lane;
        qg[n] = gp[c];
        qu[n] = up[c];
        const size_t so = (size_t)(c / CPR) * CPR + ((c % CPR) & ~3);
        sg[n] = *reinterpret_cast<const uint2*>(gsb + so);
        su[n] = *reinterpret_cast<const uint2*>(usb + so);
      }
      Slice8 xs[XS][4];
      const uint4* xp = reinterpret_cast<const uint4*>(a.x);
#pragma unroll
      for (int s = 0; s < XS; ++s) {
        const int c = CPR > 64 ? 64 * s + lane : lane % CPR;
        const int base = 128 * (c >> 2) + 8 * (c & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) xs[s][j] = make_slice_bf16(xp[(base + 32 * j) >> 3]);
      }
      float* hout = a.h + (size_t)slot * F;
      float ag = 0.f, au = 0.f;
#pragma unroll
      for (int n = 0; n < NL; ++n) {
        const int s = CPR > 64 ? n % XS : 0;
        ag += dot_piece(qg[n], xs[s], sg[n]);
        au += dot_piece(qu[n], xs[s], su[n]);
        if (n % LPRG == LPRG - 1) {
          if constexpr (CPR >= 64) {
            const float g = wave_sum(ag), u = wave_sum(au);
            if (lane == 0) store_coherent(hout + (c0 + 64 * n) / CPR, wj * silu(g) * u);
          } else {
            const float g = seg_sum<(CPR < 64 ? CPR : 64)>(ag), u = seg_sum<(CPR < 64 ? CPR : 64)>(au);
            if (lane % CPR == 0) store_coherent(hout + (c0 + 64 * n + lane) / CPR, wj * silu(g) * u);
          }
          ag = au = 0.f;
        }
      }
    }
  }
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) store_coherent_u32(a.flags + blockIdx.x, tag);

  // ---------------------------------------------------------------- down
  if (wid == 0) {
    poll_flags(a.flags, G, tag, lane, a.error);
    if (blockIdx.x == 0 && lane == 0) store_coherent_u32(a.epoch, tag);  // every workgroup has read it
  }
  __syncthreads();
  {
    // all loads first (one round trip), then the LDS stores
    constexpr int NH = (KP * F / 2 + 255) / 256;
    const int nh2 = k * F / 2;
    const unsigned long long* hsrc = reinterpret_cast<const unsigned long long*>(a.h);
    unsigned long long hv[NH];
#pragma unroll
    for (int m = 0; m < NH; ++m) hv[m] = load_coherent(hsrc + min((int)threadIdx.x + 256 * m, nh2 - 1));
#pragma unroll
    for (int m = 0; m < NH; ++m) {
      const int j = threadIdx.x + 256 * m;
      if (j < nh2) {
        s_h[2 * j] = __uint_as_float((uint32_t)hv[m]);
        s_h[2 * j + 1] = __uint_as_float((uint32_t)(hv[m] >> 32));
      }
    }
  }
  __syncthreads();
  if (has_down) {
    Slice8 hh[LPRD][4], hl[LPRD][4];
#pragma unroll
    for (int m = 0; m < LPRD; ++m) {
      const int base = 128 * (cc[m] >> 2) + 8 * (cc[m] & 3);
      const float* hs = s_h + (act[m] ? dslot[m] : 0) * F;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 lo4 = *reinterpret_cast<const float4*>(hs + base + 32 * j);
        const float4 hi4 = *reinterpret_cast<const float4*>(hs + base + 32 * j + 4);
        const bool on = act[m];
        float v[8];
        v[0] = on ? lo4.x : 0.f, v[1] = on ? lo4.y : 0.f, v[2] = on ? lo4.z : 0.f, v[3] = on ? lo4.w : 0.f;
        v[4] = on ? hi4.x : 0.f, v[5] = on ? hi4.y : 0.f, v[6] = on ? hi4.z : 0.f, v[7] = on ? hi4.w : 0.f;
        make_slice_hilo(v, hh[m][j], hl[m][j]);
      }
    }
    float acc = 0.f;
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int m = n % LPRD;
      acc += dot_piece_hilo(qd[n], hh[m], hl[m], sd[n]);
      if (n % LPRD == LPRD - 1) {
        if constexpr (P >= 64) {
          const float v = wave_sum(acc);
          if (lane == 0) a.y[r0 + n / LPRD] = v;
        } else {
          const float v = seg_sum<(P < 64 ? P : 64)>(acc);
          if (lane % P == 0) a.y[r0 + n * RPLD + lane / P] = v;
        }
        acc = 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------- host side

template <int D, int F, int KP, int EPL, int RW>
static hipError_t layer_launch(const FusedArgs& a, int G, hipStream_t s) {
  const size_t lds = (size_t)a.k * F * sizeof(float);
  hipLaunchKernelGGL((k_layer<D, F, KP, EPL, RW>), dim3(G), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int D, int F, int KP, int EPL>
static hipError_t layer_rw(const FusedArgs& a, int G, int rw, hipStream_t s) {
  if constexpr (D >= 1024) {
    if (rw == 4) return layer_launch<D, F, KP, EPL, 4>(a, G, s);
  }
  return layer_launch<D, F, KP, EPL, 1>(a, G, s);
}

template <int D, int F, int KP>
static hipError_t layer_epl(const FusedArgs& a, int G, int rw, hipStream_t s) {
  if (a.E <= 64) return layer_rw<D, F, KP, 1>(a, G, rw, s);
  if (a.E <= 128) return layer_rw<D, F, KP, 2>(a, G, rw, s);
  return layer_rw<D, F, KP, 4>(a, G, rw, s);
}

template <int D, int F>
static hipError_t layer_kp(const FusedArgs& a, int G, int rw, hipStream_t s) {
  const int k = a.k;
  if (k <= 1) return layer_epl<D, F, 1>(a, G, rw, s);
  if (k <= 2) return layer_epl<D, F, 2>(a, G, rw, s);
  if (k <= 4) return layer_epl<D, F, 4>(a, G, rw, s);
  if (k <= 8) return layer_epl<D, F, 8>(a, G, rw, s);
  return layer_epl<D, F, 16>(a, G, rw, s);
}

// Work each wave takes in the fused kernel must fit one unit per wave.
static bool fits(int d, int f, int E, int k, int G, int& rw) {
  const int W = 4 * G;
  const int cpr = d / 32, cprf = f / 32;
  if ((long)k * f * cpr / 256 > W) return false;  // gate/up units (4 pieces per lane)
  int kp = 1;
  while (kp < k) kp <<= 1;
  const int P = kp * cprf;
  const int lprd = P > 64 ? P / 64 : 1, rpld = P < 64 ? 64 / P : 1;
  const int nld = lprd > 4 ? lprd : 4;
  const int rows_w = (nld / lprd) * rpld;
  if (d / rows_w > W) return false;
  if ((size_t)k * f * sizeof(float) > 64 * 1024) return false;
  if (E > 256) return false;
  rw = (d >= 1024 && E <= G) ? 4 : 1;
  if (E * rw > W) return false;
  return true;
}

bool fused_layer_supported(int d, int f, int E, int k, int G) {
  int rw;
  if (!((d == 256 && f == 128) || (d == 2048 && f == 512))) return false;
  return fits(d, f, E, k, G, rw);
}

int fused_grid() {
  static int g = 0;
  if (!g) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 0;
    g = cus > kMaxFusedGrid ? kMaxFusedGrid : cus & ~1;  // even: flags are polled in pairs
  }
  return g;
}

hipError_t launch_layer_fused(const FusedArgs& a, int d, int f, hipStream_t s) {
  const int G = fused_grid();
  int rw;
  if (G <= 0 || !fits(d, f, a.E, a.k, G, rw)) return hipErrorInvalidValue;
  if (d == 256 && f == 128) return layer_kp<256, 128>(a, G, rw, s);
  if (d == 2048 && f == 512) return layer_kp<2048, 512>(a, G, rw, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
