// kernels_lmhead.hip -- 4-bit output layer GEMV with a fused argmax (gfx950).
//
// The pages single out the output layer: about 150,000 rows, about an eighth
// of the per-token work, stored in 4 bits ("Flint 40B: Best Mid Sized LLM",
// transcript 03:36-05:39; mirrorspeed.com page, section "Quantization").
// Decoding takes the largest logit, so the logits are reduced to one
// (value, row) pair per workgroup inside the kernel and never stored.
//
// Layout of the work: a persistent grid of G workgroups walks the matrix in
// tiles of 64*NL consecutive 16-byte pieces per wave (one piece per lane per
// load, activations of up to BP rows of x in registers).  Each workgroup
// writes its best (value, row) per x row as a 64-bit key; the last workgroup
// to arrive reduces the G keys, writes token and max logit, and clears the
// arrival counter so the next call starts from zero.
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace moe {

// Larger logit first, then the smaller row.
__device__ __forceinline__ unsigned long long make_key(float z, uint32_t row) {
  return ((unsigned long long)ordered_bits(z) << 32) | (unsigned long long)(0xFFFFFFFFu - row);
}

constexpr int kLmMaxGrid = 4096;

template <int CPR, int BP, int NL>
__global__ __launch_bounds__(256) void k_lmhead(const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                                                int V, const uint16_t* __restrict__ x, int B,
                                                unsigned long long* __restrict__ partial,
                                                unsigned* __restrict__ counter, int32_t* __restrict__ token,
                                                float* __restrict__ max_logit) {
  constexpr int D = CPR * 32;
  constexpr int XS = CPR > 64 ? CPR / 64 : 1;
  constexpr int LPR = CPR > 64 ? CPR / 64 : 1;
  static_assert(NL % LPR == 0, "a wave tile must cover whole rows");
  __shared__ unsigned long long s_best[4][BP];
  __shared__ bool s_last;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const size_t total = (size_t)V * CPR;
  const uint4* wp = reinterpret_cast<const uint4*>(wq);

  Slice8 xs[BP][XS][4];
#pragma unroll
  for (int b = 0; b < BP; ++b)
#pragma unroll
    for (int s = 0; s < XS; ++s) {
      const int cc = CPR > 64 ? 64 * s + lane : lane % CPR;
      const int base = 128 * (cc >> 2) + 8 * (cc & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (b < B)
          xs[b][s][j] = make_slice_bf16(reinterpret_cast<const uint4*>(x + (size_t)b * D)[(base + 32 * j) >> 3]);
        else
          xs[b][s][j] = Slice8{0u, 0u, 0u, 0u, 0.f};
      }
    }

  float best[BP];
  uint32_t brow[BP];
#pragma unroll
  for (int b = 0; b < BP; ++b) best[b] = -INFINITY, brow[b] = 0xFFFFFFFFu;

  for (size_t tile = (size_t)blockIdx.x * 4 + wid; tile * 64 * NL < total; tile += (size_t)gridDim.x * 4) {
    const size_t c0 = tile * 64 * NL;
    uint4 q[NL];
    uint2 sc[NL];
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const size_t c = c0 + 64 * n + lane;
      if (c < total) {
        q[n] = wp[c];
        const size_t row = c / CPR;
        const int cc = (int)(c % CPR);
        sc[n] = *reinterpret_cast<const uint2*>(ws + row * CPR + (cc & ~3));
      } else {
        q[n] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        sc[n] = make_uint2(0, 0);
      }
    }
    float acc[BP];
#pragma unroll
    for (int b = 0; b < BP; ++b) acc[b] = 0.f;
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const int s = CPR > 64 ? n % XS : 0;
#pragma unroll
      for (int b = 0; b < BP; ++b) acc[b] += dot_piece(q[n], xs[b][s], sc[n]);
      if (n % LPR == LPR - 1) {
        const size_t c = c0 + 64 * n + lane;
        const uint32_t row = (uint32_t)((CPR >= 64 ? c0 + 64 * n : c) / CPR);
#pragma unroll
        for (int b = 0; b < BP; ++b) {
          const float z = CPR >= 64 ? wave_sum(acc[b]) : seg_sum<(CPR < 64 ? CPR : 64)>(acc[b]);
          if (row < (uint32_t)V && z > best[b]) best[b] = z, brow[b] = row;
          acc[b] = 0.f;
        }
      }
    }
  }

  // wave argmax, then across the 4 waves through LDS
#pragma unroll
  for (int b = 0; b < BP; ++b) {
    float v = best[b];
    int r = (int)brow[b];  // 0xFFFFFFFF (no row) reads as -1 and loses below
    if (r < 0) v = -INFINITY, r = 0x7FFFFFFF;
    wave_argmax(v, r);
    if (lane == 0) s_best[wid][b] = r == 0x7FFFFFFF ? 0ull : make_key(v, (uint32_t)r);
  }
  __syncthreads();
  if (threadIdx.x < BP) {
    unsigned long long kmax = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) kmax = s_best[w][threadIdx.x] > kmax ? s_best[w][threadIdx.x] : kmax;
    store_coherent(partial + (size_t)blockIdx.x * BP + threadIdx.x, kmax);
    wait_vm();
  }
  __syncthreads();
  if (threadIdx.x == 0) s_last = arrive(counter) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  // last workgroup: reduce G keys per x row
  for (int b = 0; b < B; ++b) {
    unsigned long long kmax = 0;
    for (int g = threadIdx.x; g < (int)gridDim.x; g += 256) {
      const unsigned long long kv = load_coherent(partial + (size_t)g * BP + b);
      kmax = kv > kmax ? kv : kmax;
    }
    // 64-bit max over the workgroup through LDS
    __shared__ unsigned long long s_red[256];
    s_red[threadIdx.x] = kmax;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) s_red[threadIdx.x] = s_red[threadIdx.x + w] > s_red[threadIdx.x] ? s_red[threadIdx.x + w]
                                                                                            : s_red[threadIdx.x];
      __syncthreads();
    }
    if (threadIdx.x == 0) s_best[0][0] = s_red[0];
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned long long m = s_best[0][0];
      token[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFull));
      if (max_logit) max_logit[b] = unordered_bits((uint32_t)(m >> 32));
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) *counter = 0u;
}

size_t lmhead_workspace_bytes(int V, int d, int B) {
  (void)V;
  (void)d;
  const int launches = (B + 7) / 8;
  return (size_t)launches * (256 + (size_t)kLmMaxGrid * 8 * sizeof(unsigned long long));
}

static int lm_grid() {
  static int g = 0;
  if (!g) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess || cus <= 0)
      cus = 256;
    g = cus * 4 > kLmMaxGrid ? kLmMaxGrid : cus * 4;
  }
  return g;
}

template <int CPR, int BP>
static void lm_inst(const uint8_t* wq, const uint16_t* ws, int V, const uint16_t* x, int B, unsigned char* wsp,
                    int32_t* token, float* max_logit, hipStream_t s) {
  constexpr int NL = BP <= 2 ? 8 : 4;
  unsigned* counter = reinterpret_cast<unsigned*>(wsp);
  unsigned long long* partial = reinterpret_cast<unsigned long long*>(wsp + 256);
  const size_t tiles = ((size_t)V * CPR + 64 * NL - 1) / (64 * NL);
  int grid = lm_grid();
  if ((size_t)grid * 4 > tiles) grid = (int)((tiles + 3) / 4);
  hipLaunchKernelGGL((k_lmhead<CPR, BP, NL>), dim3(grid), dim3(256), 0, s, wq, ws, V, x, B, partial, counter, token,
                     max_logit);
}

template <int CPR>
static void lm_b(const uint8_t* wq, const uint16_t* ws, int V, const uint16_t* x, int B, unsigned char* wsp,
                 int32_t* token, float* max_logit, hipStream_t s) {
  if (B <= 1)
    lm_inst<CPR, 1>(wq, ws, V, x, B, wsp, token, max_logit, s);
  else if (B <= 2)
    lm_inst<CPR, 2>(wq, ws, V, x, B, wsp, token, max_logit, s);
  else if (B <= 4)
    lm_inst<CPR, 4>(wq, ws, V, x, B, wsp, token, max_logit, s);
  else
    lm_inst<CPR, 8>(wq, ws, V, x, B, wsp, token, max_logit, s);
}

hipError_t launch_lmhead(const uint8_t* wq, const uint16_t* ws, int V, int d, const uint16_t* x, int B,
                         int32_t* token, float* max_logit, void* workspace, hipStream_t s) {
  unsigned char* wsp = static_cast<unsigned char*>(workspace);
  const size_t per = 256 + (size_t)kLmMaxGrid * 8 * sizeof(unsigned long long);
  for (int b0 = 0; b0 < B; b0 += 8) {
    const int nb = B - b0 < 8 ? B - b0 : 8;
    const uint16_t* xb = x + (size_t)b0 * d;
    int32_t* tb = token + b0;
    float* mb = max_logit ? max_logit + b0 : nullptr;
    unsigned char* w = wsp + (size_t)(b0 / 8) * per;
    switch (d / 32) {
      case 8: lm_b<8>(wq, ws, V, xb, nb, w, tb, mb, s); break;
      case 16: lm_b<16>(wq, ws, V, xb, nb, w, tb, mb, s); break;
      case 32: lm_b<32>(wq, ws, V, xb, nb, w, tb, mb, s); break;
      case 64: lm_b<64>(wq, ws, V, xb, nb, w, tb, mb, s); break;
      case 128: lm_b<128>(wq, ws, V, xb, nb, w, tb, mb, s); break;
      case 256: lm_b<256>(wq, ws, V, xb, nb, w, tb, mb, s); break;
      default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
