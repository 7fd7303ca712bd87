// kernels_moe.hip -- the decode step of a 4-bit MoE layer for T tokens on gfx950.
//
// Four kernels per call:
//   router  : logits = W_r x (+b), one router row per wave, four rows per
//             workgroup.  The last workgroup to finish a token does that
//             token's softmax + top-k in one wave; the last token to finish
//             sorts the T*k (token, slot) assignments by expert (a stable
//             counting sort built from wave ballots).  Workgroup 0 of each
//             token also writes the token's activations in MFMA operand
//             order, with their per-group offset corrections.  In the stack
//             the router applies the pre-norm (RMSNorm) to the residual.
//   gate/up : per chosen expert, int4 x bf16 MFMA tiles over all the
//             tokens routed to it, so each chosen expert's weights are read
//             once per call however many tokens chose it; SwiGLU; h = w_j
//             silu(g) u stored as fp16 operands of the down step.
//   down    : the same over W_d; each assignment's o_{t,j} in fp32.
//   combine : y_t = sum_j o_{t,j} in slot order (deterministic); in the
//             stack the residual add is folded in.
// The pages describe the step: per token a small router picks a few of 256
// routed experts and only those run ("Flint 40B: Best Mid Sized LLM",
// transcript 02:35); kernels for low-bit projections, MoE routing and
// prompt processing are named in the same source (06:11).
//
// MFMA operands.  v_mfma_f32_16x16x32_{bf16,f16}: lane l supplies row l%16
// of A and column l%16 of B, each with the 8 consecutive k of chunk l/16;
// lane l receives D[4*(l/16)+v][l%16], v = 0..3.  A holds 16 tokens'
// activations, B 16 weight rows, so every lane ends with one weight row and
// four tokens, and one group scale per lane applies to all four.  One dword
// of stored codes is the 8 elements of one chunk; its 8 operand values come
// out of the magic-number conversion in the order e = 0,4,1,5,2,6,3,7 with
// the odd e scaled (see device_common.h), and the activation operands are
// stored in that same order, odd e divided by 8 (bf16) or 16 (fp16).  The
// per-group offset correction times the scale is added by one fp32 MFMA
// (16x16x4) per four groups.
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"
#include "topk.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------- top-k

__device__ __forceinline__ void store_coherent_i32(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent_i32(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// This wave's LDS operations have completed (and act as a compiler barrier).
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Softmax + top-k of one token's E logits in one wave (topk.h); lane r < k
// writes choice r.  The chosen indices are read by another workgroup of the
// same launch (the sort), so they are written coherently.
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
    store_coherent_i32(sel_idx + lane, se);
    sel_w[lane] = sw;
    if (idx_out) idx_out[lane] = se;
    if (w_out) w_out[lane] = sw;
  }
}

// ----------------------------------------------------------------- sort

// Lanes among `valid` whose expert index equals this lane's (E <= 1024).
__device__ __forceinline__ uint64_t same_expert_lanes(int e, uint64_t valid) {
  uint64_t m = valid;
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __builtin_amdgcn_ballot_w64(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// One wave: the Tk = T*k assignments a = t*k + j (chosen expert sel[a])
// grouped by expert, ascending a within an expert:
//   off[e] .. off[e+1]-1  positions of expert e in asg (off[E] = Tk)
//   asg[p]                the assignment at position p
//   act[0 .. meta[0]-1]   the experts with at least one assignment, ascending
// cnt: LDS [E]; sums: LDS [128].
__device__ void sort_by_expert(const int32_t* sel, int Tk, int E, int* cnt, int* sums, int32_t* off,
                               int32_t* act, int32_t* meta, int32_t* asg, int lane) {
  for (int i = lane; i < E; i += 64) cnt[i] = 0;
  lds_wait();
  for (int c = 0; c < Tk; c += 64) {  // counts
    const int a = c + lane;
    const bool v = a < Tk;
    const int e = v ? min(max(load_coherent_i32(sel + a), 0), E - 1) : 0;
    const uint64_t same = same_expert_lanes(e, __builtin_amdgcn_ballot_w64(v));
    if (v && lane == __builtin_ctzll(same)) cnt[e] += __builtin_popcountll(same);
    lds_wait();
  }
  // exclusive scans over experts of the counts and of the active flags
  const int per = (E + 63) / 64;
  const int e0 = min(lane * per, E), e1 = min(e0 + per, E);
  int s = 0, na = 0;
  for (int e = e0; e < e1; ++e) {
    s += cnt[e];
    na += cnt[e] > 0;
  }
  sums[lane] = s;
  sums[64 + lane] = na;
  lds_wait();
  int base = 0, abase = 0;
  for (int l = 0; l < lane; ++l) {
    base += sums[l];
    abase += sums[64 + l];
  }
  for (int e = e0; e < e1; ++e) {
    const int n = cnt[e];
    off[e] = base;
    if (n > 0) act[abase++] = e;
    cnt[e] = base;  // from here on: the next free position of expert e
    base += n;
  }
  if (lane == 63) {
    off[E] = base;
    meta[0] = abase;
  }
  lds_wait();
  for (int c = 0; c < Tk; c += 64) {  // placement, stable in a
    const int a = c + lane;
    const bool v = a < Tk;
    const int e = v ? min(max(load_coherent_i32(sel + a), 0), E - 1) : 0;
    const uint64_t same = same_expert_lanes(e, __builtin_amdgcn_ballot_w64(v));
    const int rank = __builtin_popcountll(same & ((1ull << lane) - 1ull));
    const int pos = v ? cnt[e] : 0;
    lds_wait();
    if (v) asg[pos + rank] = a;
    if (v && lane == __builtin_ctzll(same)) cnt[e] = pos + __builtin_popcountll(same);
    lds_wait();
  }
}

// ----------------------------------------------------------------- router

// grid (ceil(E/4), T), block 256: wave w of workgroup b computes logit
// 4b + w of token t.  EPL = experts per lane in the top-k wave, ceil(E/64).
template <int D, int EPL>
__global__ __launch_bounds__(256) void k_router(const LayerArgs a, const uint16_t* __restrict__ x,
                                                const float* __restrict__ resid, float eps, int T,
                                                int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                                uint16_t* __restrict__ x_trace) {
  constexpr int NI = D / 256;  // float4 columns per lane: 4*lane + 256*i
  constexpr int G = D / 32;
  __shared__ int s_cnt[1024];
  __shared__ int s_sums[128];
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave, t = blockIdx.y;
  const bool row_ok = e < a.E;
  const float4* wrow = reinterpret_cast<const float4*>(a.router_w + (size_t)min(e, a.E - 1) * D);
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
      if (x_trace && blockIdx.x == 0 && wave == 0)
        reinterpret_cast<uint2*>(x_trace + (size_t)t * D)[64 * i + lane] =
            make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    }
  }

  if (blockIdx.x == 0 && wave == 0) {
    // The token's MFMA operand row: chunk of 8 elements stored as
    // (x0, x4, x1/8, x5/8, x2, x6, x3/8, x7/8); lane 2m holds x0..x3 of a
    // chunk and lane 2m+1 holds x4..x7, so neighbours trade halves.  Per
    // group of 32 (8 lanes): corr = -136 * sum(even e) - 24 * sum(odd e).
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float o0 = dpp_f<kDppXor1>(xv[i][0]), o1 = dpp_f<kDppXor1>(xv[i][1]);
      const float o2 = dpp_f<kDppXor1>(xv[i][2]), o3 = dpp_f<kDppXor1>(xv[i][3]);
      uint2 pk;
      if ((lane & 1) == 0) {
        pk.x = pack_bf16(xv[i][0], o0);
        pk.y = pack_bf16(xv[i][1] * 0.125f, o1 * 0.125f);
      } else {
        pk.x = pack_bf16(o2, xv[i][2]);
        pk.y = pack_bf16(o3 * 0.125f, xv[i][3] * 0.125f);
      }
      reinterpret_cast<uint2*>(a.xp + (size_t)t * D)[64 * i + lane] = pk;
      const float cr = seg_sum<8>(-136.0f * (xv[i][0] + xv[i][2]) - 24.0f * (xv[i][1] + xv[i][3]));
      if ((lane & 7) == 0) a.corr_x[(size_t)t * G + (256 * i + 4 * lane) / 32] = cr;
    }
  }

  if (row_ok) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      acc = fmaf(w[i].x, xv[i][0], acc);
      acc = fmaf(w[i].y, xv[i][1], acc);
      acc = fmaf(w[i].z, xv[i][2], acc);
      acc = fmaf(w[i].w, xv[i][3], acc);
    }
    acc = wave_sum(acc);
    if (a.router_b) acc += a.router_b[e];
    if (lane == 0) store_coherent(a.logits + (size_t)t * a.E + e, acc);
  }

  // Arrival: the last workgroup of token t selects its experts.
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) s_last = arrive(&a.counters[t]) == gridDim.x - 1;
  __syncthreads();
  if (!s_last || wave != 0) return;
  int32_t* io = idx_out ? idx_out + (size_t)t * a.k : nullptr;
  float* wo = w_out ? w_out + (size_t)t * a.k : nullptr;
  topk_wave<EPL>(a.logits + (size_t)t * a.E, a.E, a.k, a.norm_topk, lane, a.sel_idx + t * a.k,
                 a.sel_w + t * a.k, io, wo);
  wait_vm();
  unsigned prev = 0;
  if (lane == 0) {
    a.counters[t] = 0u;  // ready for the next call
    prev = arrive(a.tokens_done);
  }
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev != (unsigned)(T - 1)) return;
  // the last token: group the assignments by expert
  sort_by_expert(a.sel_idx, T * a.k, a.E, s_cnt, s_sums, a.off, a.act, a.meta, a.asg, lane);
  if (lane == 0) *a.tokens_done = 0u;
}

// ----------------------------------------------------------------- MFMA tiles

// B operand of one MFMA from one dword of codes (8 elements of a chunk):
// bf16 128+u (even e) / 128+8u (odd e), or fp16 1024+u / 1024+16u.
__device__ __forceinline__ bf16x8_t codes_bf16(uint32_t w) {
  const uint4 v = make_uint4((w & 0x000F000Fu) | 0x43004300u, ((w >> 1) & 0x00780078u) | 0x43004300u,
                             ((w >> 8) & 0x000F000Fu) | 0x43004300u, ((w >> 9) & 0x00780078u) | 0x43004300u);
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ f16x8_t codes_f16(uint32_t w) {
  const uint32_t w8 = w >> 8;
  const uint4 v = make_uint4((w & 0x000F000Fu) | 0x64006400u, (w & 0x00F000F0u) | 0x64006400u,
                             (w8 & 0x000F000Fu) | 0x64006400u, (w8 & 0x00F000F0u) | 0x64006400u);
  return __builtin_bit_cast(f16x8_t, v);
}

__device__ __forceinline__ uint32_t dword_of(uint4 v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }
// binary16 scale j (0..3) of the four packed in sc
__device__ __forceinline__ float scale_of(uint2 sc, int j) {
  const uint32_t d = (j & 2) ? sc.y : sc.x;
  return f16_bits_to_f32((j & 1) ? (d >> 16) : (d & 0xFFFFu));
}

template <bool HALF>
__device__ __forceinline__ f32x4_t mfma_group(uint4 act, uint32_t codes) {
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  if constexpr (HALF)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, act), codes_f16(codes), z, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, act), codes_bf16(codes), z, 0, 0,
                                                   0);
}

// Contraction of one wave's share of K for TPW weight tiles (16 rows each)
// against up to two token tiles.
//   K      contraction length (elements); KSPLIT waves share it, each taking
//          GW = K/32/KSPLIT consecutive groups (a multiple of 4)
//   wrow   per tile: this lane's weight row (stored codes) and its scales
//   opnd   operand rows ([row][K] in operand order) and corr ([row][K/32]);
//          the lane's token of tile tt is row orow[tt], used when ov[tt]
template <int K, int KSPLIT, bool HALF>
__device__ __forceinline__ void contract(f32x4_t (&acc)[KSPLIT][2], const uint8_t* const (&wrow)[KSPLIT],
                                         const uint16_t* const (&srow)[KSPLIT], const uint16_t* __restrict__ opnd,
                                         const float* __restrict__ corr, const int (&orow)[2], const bool (&ov)[2],
                                         int ntt, int kpart, int lane) {
  constexpr int G = K / 32;
  constexpr int BW = G / KSPLIT / 4;  // 128-element blocks per wave
  constexpr int NB = BW < 2 ? BW : 2; // blocks per pass
  static_assert(BW >= 1 && BW % NB == 0, "each wave takes whole blocks");
  const int q = lane >> 4;
  for (int ps = 0; ps < BW / NB; ++ps) {
    const int kb0 = kpart * BW + ps * NB;
    uint4 wq[KSPLIT][NB];
    uint2 sc[KSPLIT][NB];
#pragma unroll
    for (int i = 0; i < KSPLIT; ++i)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        wq[i][b] = *reinterpret_cast<const uint4*>(wrow[i] + (size_t)(kb0 + b) * 64 + 16 * q);
        sc[i][b] = *reinterpret_cast<const uint2*>(srow[i] + 4 * (kb0 + b));
      }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt >= ntt) break;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint16_t* op = opnd + (size_t)orow[tt] * K + (kb0 + b) * 128 + 8 * q;
        uint4 xf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xf[j] = ov[tt] ? *reinterpret_cast<const uint4*>(op + 32 * j) : make_uint4(0u, 0u, 0u, 0u);
        const float cx = ov[tt] ? corr[(size_t)orow[tt] * G + 4 * (kb0 + b) + q] : 0.f;
#pragma unroll
        for (int i = 0; i < KSPLIT; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4_t c = mfma_group<HALF>(xf[j], dword_of(wq[i][b], j));
            const float s = scale_of(sc[i][b], j);
            acc[i][tt][0] = fmaf(s, c[0], acc[i][tt][0]);
            acc[i][tt][1] = fmaf(s, c[1], acc[i][tt][1]);
            acc[i][tt][2] = fmaf(s, c[2], acc[i][tt][2]);
            acc[i][tt][3] = fmaf(s, c[3], acc[i][tt][3]);
          }
          // sum over the block's 4 groups of corr(token, g) * scale(row, g)
          acc[i][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(cx, scale_of(sc[i][b], q), acc[i][tt], 0, 0, 0);
        }
      }
    }
  }
}

// ----------------------------------------------------------------- gate/up

// Work item: (active expert, 32 rows of f).  KSPLIT waves share K = d and
// 4/KSPLIT share the 4 weight tiles (gate rows 0-15, 16-31, up rows 0-15,
// 16-31); tokens in chunks of 32.  Partial tiles meet in LDS, then 128
// threads form h for (token, 8 rows) each and store it as an fp16 operand
// chunk, with the group's offset correction.
template <int D>
__global__ __launch_bounds__(256) void k_gateup(const LayerArgs a) {
  constexpr int G = D / 32;
  constexpr int KSPLIT = G / 4 >= 4 ? 4 : G / 4;
  constexpr int TPW = KSPLIT;  // tiles per wave
  __shared__ float P[KSPLIT][4][2][16][16];
  const int f = a.f, k = a.k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15;
  const int kpart = wave % KSPLIT, rpart = wave / KSPLIT;
  const int rbs = f / 32;
  const int nitems = a.meta[0] * rbs;
  const size_t mq = (size_t)f * (D / 2), ms = (size_t)f * G;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int ai = item / rbs, rb = item - ai * rbs;
    const int e = a.act[ai];
    const int p0 = a.off[e], n = a.off[e + 1] - p0;
    const uint8_t* wrow[TPW];
    const uint16_t* srow[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int wt = rpart * TPW + i;
      const int row = rb * 32 + 16 * (wt & 1) + r16;
      wrow[i] = (wt < 2 ? a.gate_q : a.up_q) + e * mq + (size_t)row * (D / 2);
      srow[i] = (wt < 2 ? a.gate_s : a.up_s) + e * ms + (size_t)row * G;
    }
    for (int tc = 0; tc < n; tc += 32) {
      const int ntt = n - tc > 16 ? 2 : 1;
      int orow[2];
      bool ov[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int pt = tc + 16 * tt + r16;
        ov[tt] = pt < n;
        orow[tt] = ov[tt] ? a.asg[p0 + pt] / k : 0;
      }
      f32x4_t acc[TPW][2];
#pragma unroll
      for (int i = 0; i < TPW; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      contract<D, KSPLIT, false>(acc, wrow, srow, a.xp, a.corr_x, orow, ov, ntt, kpart, lane);
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          *reinterpret_cast<f32x4_t*>(&P[kpart][rpart * TPW + i][tt][r16][4 * (lane >> 4)]) = acc[i][tt];
      __syncthreads();
      if (threadIdx.x < 128) {
        const int c = threadIdx.x >> 2, m = threadIdx.x & 3;  // token of the chunk, 8-row chunk
        const int tt = c >> 4, cc = c & 15;
        const int pt = tc + c;
        const bool valid = pt < n;
        const float wj = valid ? a.sel_w[a.asg[p0 + pt]] : 0.f;
        float hv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * m + i, wt = r >> 4, rr = r & 15;
          float g = 0.f, u = 0.f;
#pragma unroll
          for (int kp = 0; kp < KSPLIT; ++kp) {
            g += P[kp][wt][tt][rr][cc];
            u += P[kp][2 + wt][tt][rr][cc];
          }
          hv[i] = wj * silu(g) * u;
        }
        uint4 o;
        o.x = pack_f16(hv[0], hv[4]);
        o.y = pack_f16(hv[1] * 0.0625f, hv[5] * 0.0625f);
        o.z = pack_f16(hv[2], hv[6]);
        o.w = pack_f16(hv[3] * 0.0625f, hv[7] * 0.0625f);
        const float ev = (f16_lo(o.x) + f16_hi(o.x)) + (f16_lo(o.z) + f16_hi(o.z));
        const float od = (f16_lo(o.y) + f16_hi(o.y)) + (f16_lo(o.w) + f16_hi(o.w));
        const float cr = seg_sum<4>(-1032.0f * ev - 1152.0f * od);
        if (valid) {
          *reinterpret_cast<uint4*>(a.h16 + (size_t)(p0 + pt) * f + rb * 32 + 8 * m) = o;
          if (m == 0) a.corr_h[(size_t)(p0 + pt) * (f / 32) + rb] = cr;
        }
      }
      __syncthreads();
    }
  }
}

// ----------------------------------------------------------------- down

// Work item: (active expert, 64 rows of d) = 4 weight tiles; K = f.  The
// summed tiles give o_{t,j} for every assignment of the expert, written to
// obuf[t*k + j][row].
template <int F>
__global__ __launch_bounds__(256) void k_down(const LayerArgs a) {
  constexpr int G = F / 32;
  constexpr int KSPLIT = G / 4 >= 4 ? 4 : G / 4;
  constexpr int TPW = KSPLIT;
  __shared__ float P[KSPLIT][4][2][16][16];
  const int d = a.d;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15;
  const int kpart = wave % KSPLIT, rpart = wave / KSPLIT;
  const int rbs = d / 64;
  const int nitems = a.meta[0] * rbs;
  const size_t mq = (size_t)d * (F / 2), ms = (size_t)d * G;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int ai = item / rbs, rb = item - ai * rbs;
    const int e = a.act[ai];
    const int p0 = a.off[e], n = a.off[e + 1] - p0;
    const uint8_t* wrow[TPW];
    const uint16_t* srow[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int row = rb * 64 + 16 * (rpart * TPW + i) + r16;
      wrow[i] = a.down_q + e * mq + (size_t)row * (F / 2);
      srow[i] = a.down_s + e * ms + (size_t)row * G;
    }
    for (int tc = 0; tc < n; tc += 32) {
      const int ntt = n - tc > 16 ? 2 : 1;
      int orow[2];
      bool ov[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int pt = tc + 16 * tt + r16;
        ov[tt] = pt < n;
        orow[tt] = ov[tt] ? p0 + pt : 0;
      }
      f32x4_t acc[TPW][2];
#pragma unroll
      for (int i = 0; i < TPW; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      contract<F, KSPLIT, true>(acc, wrow, srow, a.h16, a.corr_h, orow, ov, ntt, kpart, lane);
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          *reinterpret_cast<f32x4_t*>(&P[kpart][rpart * TPW + i][tt][r16][4 * (lane >> 4)]) = acc[i][tt];
      __syncthreads();
      {
        const int c = threadIdx.x >> 3, m = threadIdx.x & 7;  // token of the chunk, 8 rows
        const int tt = c >> 4, cc = c & 15;
        const int pt = tc + c;
        if (pt < n) {
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 8 * m + i, wt = r >> 4, rr = r & 15;
            float s = 0.f;
#pragma unroll
            for (int kp = 0; kp < KSPLIT; ++kp) s += P[kp][wt][tt][rr][cc];
            v[i] = s;
          }
          float4* dst = reinterpret_cast<float4*>(a.obuf + (size_t)a.asg[p0 + pt] * d + rb * 64 + 8 * m);
          dst[0] = make_float4(v[0], v[1], v[2], v[3]);
          dst[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
      }
      __syncthreads();
    }
  }
}

// ----------------------------------------------------------------- combine

// y_t = sum_{j<k} o_{t,j} (slot order); with resid, resid_t += y_t.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ obuf, int T, int d, int k,
                                                 float* __restrict__ y_out, float* __restrict__ resid) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // float4 index over [T][d]
  if (i >= T * d / 4) return;
  const int t = (4 * i) / d, r = 4 * i - t * d;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float4 o = *reinterpret_cast<const float4*>(obuf + ((size_t)t * k + j) * d + r);
    s.x += o.x;
    s.y += o.y;
    s.z += o.z;
    s.w += o.w;
  }
  if (resid) {
    float4* rp = reinterpret_cast<float4*>(resid + (size_t)t * d + r);
    float4 rv = *rp;
    rv.x += s.x;
    rv.y += s.y;
    rv.z += s.z;
    rv.w += s.w;
    *rp = rv;
  }
  if (y_out) *reinterpret_cast<float4*>(y_out + (size_t)t * d + r) = s;
}

// ----------------------------------------------------------------- launchers

template <int D, int EPL>
static void router_launch(const LayerArgs& a, const uint16_t* x, const float* r, float eps, int T, int32_t* io,
                          float* wo, uint16_t* xt, hipStream_t s) {
  hipLaunchKernelGGL((k_router<D, EPL>), dim3((a.E + 3) / 4, T), dim3(256), 0, s, a, x, r, eps, T, io, wo, xt);
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

static int grid_for(int items) { return items < kMaxGroupedGrid ? items : kMaxGroupedGrid; }

hipError_t launch_gateup(const LayerArgs& a, int T, hipStream_t s) {
  const int items = (a.E < T * a.k ? a.E : T * a.k) * (a.f / 32);
  const dim3 g(grid_for(items)), b(256);
  switch (a.d) {
    case 256: hipLaunchKernelGGL((k_gateup<256>), g, b, 0, s, a); break;
    case 512: hipLaunchKernelGGL((k_gateup<512>), g, b, 0, s, a); break;
    case 1024: hipLaunchKernelGGL((k_gateup<1024>), g, b, 0, s, a); break;
    case 2048: hipLaunchKernelGGL((k_gateup<2048>), g, b, 0, s, a); break;
    case 4096: hipLaunchKernelGGL((k_gateup<4096>), g, b, 0, s, a); break;
    case 8192: hipLaunchKernelGGL((k_gateup<8192>), g, b, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_down(const LayerArgs& a, int T, hipStream_t s) {
  const int items = (a.E < T * a.k ? a.E : T * a.k) * (a.d / 64);
  const dim3 g(grid_for(items)), b(256);
  switch (a.f) {
    case 128: hipLaunchKernelGGL((k_down<128>), g, b, 0, s, a); break;
    case 256: hipLaunchKernelGGL((k_down<256>), g, b, 0, s, a); break;
    case 512: hipLaunchKernelGGL((k_down<512>), g, b, 0, s, a); break;
    case 1024: hipLaunchKernelGGL((k_down<1024>), g, b, 0, s, a); break;
    case 2048: hipLaunchKernelGGL((k_down<2048>), g, b, 0, s, a); break;
    case 4096: hipLaunchKernelGGL((k_down<4096>), g, b, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const LayerArgs& a, int T, float* y_out, float* residual, hipStream_t s) {
  const int n4 = T * a.d / 4;
  hipLaunchKernelGGL(k_combine, dim3((n4 + 255) / 256), dim3(256), 0, s, a.obuf, T, a.d, a.k, y_out, residual);
  return hipGetLastError();
}

}  // namespace moe
