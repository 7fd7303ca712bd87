// kernels_moe.hip -- the decode step of a 4-bit MoE layer for T tokens on gfx950.
//
// Four kernels per call:
//   router  : logits = W_r x (+b), one router row per wave, held in
//             registers across a block of 4 tokens.  The last workgroup to
//             finish a token block does its 4 softmax + top-k selections,
//             one wave each; the last token to finish sorts the T*k (token,
//             slot) assignments by expert (a stable counting sort built from
//             wave ballots).  Workgroup 0 also writes each token's
//             activations in MFMA operand order with their per-group offset
//             corrections.  In the stack the router applies the pre-norm
//             (RMSNorm) to the residual.
//   gate/up : one wave per (chosen expert, 16 rows, chunk of up to 32 of its
//             tokens): int4 x bf16 MFMA tiles, so each chosen expert's
//             weights are read once per call however many tokens chose it;
//             SwiGLU in registers; h = w_j silu(g) u stored as fp16 operands
//             of the down step.
//   down    : the same shape of work over W_d with int4 x fp16 MFMA; each
//             assignment's o_{t,j} in fp32.
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
// out of the magic-number conversion in the order e = 0,4,1,5,2,6,3,7 (see
// device_common.h) and the activation operands are stored in that order.
// gate/up: bf16 128+u / 128+8u against x / x/8, the offsets removed by the
// per-group correction times the scale, one fp32 MFMA (16x16x4) per four
// groups.  down: the codes become exact signed fp16 q = u - 8 with packed
// fp16 arithmetic, so h needs no correction.
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
//   act[i], i < meta[0]   the experts with at least one assignment, ascending
//   chunk_off[i]          32-token chunks of the active experts before act[i]
//                         (chunk_off[meta[0]] = all chunks)
// cnt: LDS [E]; ssel: LDS [Tk]; sums: LDS [192].
__device__ void sort_by_expert(const int32_t* sel, int Tk, int E, int* cnt, int* ssel, int* sums, int32_t* off,
                               int32_t* act, int32_t* chunk_off, int32_t* meta, int32_t* asg, int lane) {
  // the chosen experts into LDS, 8 loads in flight per lane
  for (int c0 = 0; c0 < Tk; c0 += 512) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = load_coherent_i32(sel + min(c0 + 64 * i + lane, Tk - 1));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (c0 + 64 * i + lane < Tk) ssel[c0 + 64 * i + lane] = min(max(v[i], 0), E - 1);
  }
  for (int i = lane; i < E; i += 64) cnt[i] = 0;
  lds_wait();
  for (int c = 0; c < Tk; c += 64) {  // counts
    const int a = c + lane;
    const bool v = a < Tk;
    const int e = v ? ssel[a] : 0;
    const uint64_t same = same_expert_lanes(e, __builtin_amdgcn_ballot_w64(v));
    if (v && lane == __builtin_ctzll(same)) cnt[e] += __builtin_popcountll(same);
    lds_wait();
  }
  // exclusive scans over experts: counts, active flags, chunks
  const int per = (E + 63) / 64;
  const int e0 = min(lane * per, E), e1 = min(e0 + per, E);
  int s = 0, na = 0, nc = 0;
  for (int e = e0; e < e1; ++e) {
    const int n = cnt[e];
    s += n;
    na += n > 0;
    nc += (n + 31) >> 5;
  }
  sums[lane] = s;
  sums[64 + lane] = na;
  sums[128 + lane] = nc;
  lds_wait();
  int base = 0, abase = 0, cbase = 0;
  for (int l = 0; l < lane; ++l) {
    base += sums[l];
    abase += sums[64 + l];
    cbase += sums[128 + l];
  }
  for (int e = e0; e < e1; ++e) {
    const int n = cnt[e];
    off[e] = base;
    if (n > 0) {
      act[abase] = e;
      chunk_off[abase] = cbase;
      ++abase;
      cbase += (n + 31) >> 5;
    }
    cnt[e] = base;  // from here on: the next free position of expert e
    base += n;
  }
  if (lane == 63) {
    off[E] = base;
    chunk_off[abase] = cbase;
    meta[0] = abase;
  }
  lds_wait();
  for (int c = 0; c < Tk; c += 64) {  // placement, stable in a
    const int a = c + lane;
    const bool v = a < Tk;
    const int e = v ? ssel[a] : 0;
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

constexpr int kRouterTokens = 4;  // tokens per router workgroup
constexpr int kCounterStride = 32;  // one arrival counter per 128-byte line

// grid (ceil(E/4), ceil(T/4)), block 256: wave w of workgroup (b, c) holds
// router row 4b + w in registers and computes its logit for tokens 4c ..
// 4c+3.  One arrival per workgroup on the token block's counter (own cache
// line); the last workgroup of a block does the top-k of its 4 tokens, one
// per wave; the last token overall runs the sort.  EPL = ceil(E/64).
template <int D, int EPL>
__global__ __launch_bounds__(256) void k_router(const LayerArgs a, const uint16_t* __restrict__ x,
                                                const float* __restrict__ resid, float eps, int T,
                                                int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                                uint16_t* __restrict__ x_trace) {
  constexpr int NI = D / 256;  // float4 columns per lane: 4*lane + 256*i
  constexpr int G = D / 32;
  __shared__ int s_cnt[1024];
  __shared__ int s_sel[kMaxAssignments];
  __shared__ int s_sums[192];
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  const bool row_ok = e < a.E;
  const float4* wrow = reinterpret_cast<const float4*>(a.router_w + (size_t)min(e, a.E - 1) * D);
  float4 w[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) w[i] = wrow[64 * i + lane];
  const float bias = row_ok && a.router_b ? a.router_b[e] : 0.f;

  for (int tb = 0; tb < kRouterTokens; ++tb) {
    const int t = blockIdx.y * kRouterTokens + tb;
    if (t >= T) break;
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
        if (x_trace && blockIdx.x == 0 && wave == tb)
          reinterpret_cast<uint2*>(x_trace + (size_t)t * D)[64 * i + lane] =
              make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      }
    }

    if (blockIdx.x == 0 && wave == tb) {
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
      acc = wave_sum(acc) + bias;
      if (lane == 0) store_coherent(a.logits + (size_t)t * a.E + e, acc);
    }
  }

  // Arrival: the last workgroup of this token block selects its experts.
  unsigned* counter = a.counters + blockIdx.y * kCounterStride;
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) s_last = arrive(counter) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  const int t = blockIdx.y * kRouterTokens + wave;
  if (t >= T) return;
  int32_t* io = idx_out ? idx_out + (size_t)t * a.k : nullptr;
  float* wo = w_out ? w_out + (size_t)t * a.k : nullptr;
  topk_wave<EPL>(a.logits + (size_t)t * a.E, a.E, a.k, a.norm_topk, lane, a.sel_idx + t * a.k,
                 a.sel_w + t * a.k, io, wo);
  wait_vm();
  unsigned prev = 0;
  if (lane == 0) {
    if (wave == 0) *counter = 0u;  // every workgroup of the block has arrived
    prev = arrive(a.tokens_done);
  }
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev != (unsigned)(T - 1)) return;
  // the last token: group the assignments by expert
  sort_by_expert(a.sel_idx, T * a.k, a.E, s_cnt, s_sel, s_sums, a.off, a.act, a.chunk_off, a.meta, a.asg, lane);
  if (lane == 0) *a.tokens_done = 0u;
}

// ----------------------------------------------------------------- MFMA tiles

// B operand of one MFMA from one dword of codes (8 elements of a chunk).
// bf16: 128+u (even e) / 128+8u (odd e), offsets removed afterwards with
// the activations' per-group correction.
__device__ __forceinline__ bf16x8_t codes_bf16(uint32_t w) {
  const uint4 v = make_uint4((w & 0x000F000Fu) | 0x43004300u, ((w >> 1) & 0x00780078u) | 0x43004300u,
                             ((w >> 8) & 0x000F000Fu) | 0x43004300u, ((w >> 9) & 0x00780078u) | 0x43004300u);
  return __builtin_bit_cast(bf16x8_t, v);
}
// fp16 signed codes q = u - 8, exact: (1024+u) - 1032 for even e and
// (1024+16u)/16 - 72 for odd e, with packed fp16 add / fma.
__device__ __forceinline__ f16x8_t codes_f16_signed(uint32_t w) {
  const f16x2_t off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2_t sx = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2_t so = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w8 = w >> 8;
  const f16x2_t p0 = __builtin_bit_cast(f16x2_t, (w & 0x000F000Fu) | 0x64006400u) + off;
  const f16x2_t p1 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, (w & 0x00F000F0u) | 0x64006400u), sx, so);
  const f16x2_t p2 = __builtin_bit_cast(f16x2_t, (w8 & 0x000F000Fu) | 0x64006400u) + off;
  const f16x2_t p3 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, (w8 & 0x00F000F0u) | 0x64006400u), sx, so);
  const uint4 v = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                             __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
  return __builtin_bit_cast(f16x8_t, v);
}

__device__ __forceinline__ uint32_t dword_of(uint4 v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }
// binary16 scale j (0..3) of the four packed in sc
__device__ __forceinline__ float scale_of(uint2 sc, int j) {
  const uint32_t d = (j & 2) ? sc.y : sc.x;
  return f16_bits_to_f32((j & 1) ? (d >> 16) : (d & 0xFFFFu));
}
__device__ __forceinline__ void fma4(f32x4_t& acc, float s, f32x4_t c) {
  acc[0] = fmaf(s, c[0], acc[0]);
  acc[1] = fmaf(s, c[1], acc[1]);
  acc[2] = fmaf(s, c[2], acc[2]);
  acc[3] = fmaf(s, c[3], acc[3]);
}

// Work item of one wave: (active expert, 16 weight rows, chunk of up to 32
// tokens).  Item w of an expert-major enumeration: the expert is the last
// active index i with rows * chunk_off[i] <= w (binary search in LDS);
// within it, chunks vary fastest so that the waves of a workgroup usually
// share their weight rows.
struct WaveItem {
  int e, rt, tc, p0, n;
};
__device__ __forceinline__ WaveItem wave_item(const LayerArgs& a, const int* s_cp, int nact, int rts, int w) {
  int lo = 0, hi = nact - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (rts * s_cp[mid] <= w) lo = mid; else hi = mid - 1;
  }
  const int nch = s_cp[lo + 1] - s_cp[lo];
  const int local = w - rts * s_cp[lo];
  WaveItem it;
  it.e = a.act[lo];
  it.rt = local / nch;
  it.tc = (local - it.rt * nch) * 32;
  it.p0 = a.off[it.e];
  it.n = a.off[it.e + 1] - it.p0;
  return it;
}

// ----------------------------------------------------------------- gate/up

// One wave: gate and up rows 16*rt .. 16*rt+15 of expert e for up to 32
// tokens (two token tiles), the whole of K = d streamed in 128-element
// blocks with one block of loads in flight ahead of the MFMAs.  Epilogue in
// registers: h = w_j * silu(g) * u, written as fp16 in operand order
// (0,4,1,5,2,6,3,7 within each 8 rows) for the down step.
struct GUStage {
  uint4 g, u;
  uint2 sg, su;
  uint4 x[2][4];
  float cx[2];
};

// Every load is unconditional (rows of absent tokens are clamped to a real
// one and their output rows discarded), so the compiler's count of loads in
// flight stays exact and a wait never drains the next block's loads.
template <int D>
__device__ __forceinline__ void gu_load(GUStage& st, int b, const uint8_t* gr, const uint8_t* ur,
                                        const uint16_t* gsr, const uint16_t* usr, const uint16_t* xp,
                                        const float* corr_x, const int (&trow)[2], int q) {
  st.g = *reinterpret_cast<const uint4*>(gr + b * 64 + 16 * q);
  st.u = *reinterpret_cast<const uint4*>(ur + b * 64 + 16 * q);
  st.sg = *reinterpret_cast<const uint2*>(gsr + 4 * b);
  st.su = *reinterpret_cast<const uint2*>(usr + 4 * b);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const uint16_t* op = xp + (size_t)trow[tt] * D + b * 128 + 8 * q;
#pragma unroll
    for (int j = 0; j < 4; ++j) st.x[tt][j] = *reinterpret_cast<const uint4*>(op + 32 * j);
    st.cx[tt] = corr_x[(size_t)trow[tt] * (D / 32) + 4 * b + q];
  }
}

__device__ __forceinline__ void gu_compute(const GUStage& st, f32x4_t (&acc)[2][2], int ntt, int q) {
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    if (tt >= ntt) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, st.x[tt][j]);
      const f32x4_t cg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, codes_bf16(dword_of(st.g, j)), z, 0, 0, 0);
      const f32x4_t cu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, codes_bf16(dword_of(st.u, j)), z, 0, 0, 0);
      fma4(acc[0][tt], scale_of(st.sg, j), cg);
      fma4(acc[1][tt], scale_of(st.su, j), cu);
    }
    // sum over the block's 4 groups of corr(token, g) * scale(row, g)
    acc[0][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(st.cx[tt], scale_of(st.sg, q), acc[0][tt], 0, 0, 0);
    acc[1][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(st.cx[tt], scale_of(st.su, q), acc[1][tt], 0, 0, 0);
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_gateup(const LayerArgs a) {
  constexpr int NBLK = D / 128;
  constexpr int G = D / 32;
  __shared__ int s_cp[1025];
  const int nact = a.meta[0];
  for (int i = threadIdx.x; i <= nact; i += 256) s_cp[i] = a.chunk_off[i];
  __syncthreads();
  const int f = a.f, k = a.k, rts = f / 16;
  const int total = rts * s_cp[nact];
  const int lane = threadIdx.x & 63, r16 = lane & 15, q = lane >> 4;
  const size_t mq = (size_t)f * (D / 2), ms = (size_t)f * G;
  for (int w = blockIdx.x * 4 + (threadIdx.x >> 6); w < total; w += gridDim.x * 4) {
    const WaveItem it = wave_item(a, s_cp, nact, rts, w);
    const int row = it.rt * 16 + r16;
    const uint8_t* gr = a.gate_q + it.e * mq + (size_t)row * (D / 2);
    const uint8_t* ur = a.up_q + it.e * mq + (size_t)row * (D / 2);
    const uint16_t* gsr = a.gate_s + it.e * ms + (size_t)row * G;
    const uint16_t* usr = a.up_s + it.e * ms + (size_t)row * G;
    const int ntt = it.n - it.tc > 16 ? 2 : 1;
    int trow[2];  // token of this lane's A-operand row (a real one for absent rows)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) trow[tt] = a.asg[it.p0 + min(it.tc + 16 * tt + r16, it.n - 1)] / k;
    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Two stages; the loads past the last block repeat it (unconditional
    // loads keep the compiler's wait counts exact, so a wait for one block
    // never drains the next block's loads).
    GUStage s0, s1;
    gu_load<D>(s0, 0, gr, ur, gsr, usr, a.xp, a.corr_x, trow, q);
    gu_load<D>(s1, 1, gr, ur, gsr, usr, a.xp, a.corr_x, trow, q);
    for (int b = 0; b < NBLK; b += 2) {
      gu_compute(s0, acc, ntt, q);
      gu_load<D>(s0, min(b + 2, NBLK - 1), gr, ur, gsr, usr, a.xp, a.corr_x, trow, q);
      gu_compute(s1, acc, ntt, q);
      gu_load<D>(s1, min(b + 3, NBLK - 1), gr, ur, gsr, usr, a.xp, a.corr_x, trow, q);
    }
    // lane: weight row r16, tokens 4q+v of each tile
    const int e8 = r16 & 7;
    const int col = it.rt * 16 + (r16 & 8) + 2 * (e8 & 3) + (e8 >> 2);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt >= ntt) break;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int pt = it.tc + 16 * tt + 4 * q + v;
        if (pt < it.n) {
          const float wj = a.sel_w[a.asg[it.p0 + pt]];
          const float h = wj * silu(acc[0][tt][v]) * acc[1][tt][v];
          a.h16[(size_t)(it.p0 + pt) * f + col] = __builtin_bit_cast(uint16_t, (_Float16)h);
        }
      }
    }
  }
}

// ----------------------------------------------------------------- down

// One wave: rows 16*rt .. 16*rt+15 of W_d[e] for up to 32 tokens, K = f;
// signed fp16 codes against the fp16 h operands.  o_{t,j} goes to
// obuf[t*k + j][row].
struct DStage {
  uint4 w;
  uint2 s;
  uint4 h[2][4];
};

template <int F>
__device__ __forceinline__ void dn_load(DStage& st, int b, const uint8_t* wr, const uint16_t* sr,
                                        const uint16_t* h16, const int (&prow)[2], int q) {
  st.w = *reinterpret_cast<const uint4*>(wr + b * 64 + 16 * q);
  st.s = *reinterpret_cast<const uint2*>(sr + 4 * b);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const uint16_t* op = h16 + (size_t)prow[tt] * F + b * 128 + 8 * q;
#pragma unroll
    for (int j = 0; j < 4; ++j) st.h[tt][j] = *reinterpret_cast<const uint4*>(op + 32 * j);
  }
}

__device__ __forceinline__ void dn_compute(const DStage& st, f32x4_t (&acc)[2], int ntt) {
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x8_t wb = codes_f16_signed(dword_of(st.w, j));
    const float s = scale_of(st.s, j);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt >= ntt) break;
      const f32x4_t c =
          __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, st.h[tt][j]), wb, z, 0, 0, 0);
      fma4(acc[tt], s, c);
    }
  }
}

template <int F>
__global__ __launch_bounds__(256) void k_down(const LayerArgs a) {
  constexpr int NBLK = F / 128;
  constexpr int G = F / 32;
  __shared__ int s_cp[1025];
  const int nact = a.meta[0];
  for (int i = threadIdx.x; i <= nact; i += 256) s_cp[i] = a.chunk_off[i];
  __syncthreads();
  const int d = a.d, rts = d / 16;
  const int total = rts * s_cp[nact];
  const int lane = threadIdx.x & 63, r16 = lane & 15, q = lane >> 4;
  const size_t mq = (size_t)d * (F / 2), ms = (size_t)d * G;
  for (int w = blockIdx.x * 4 + (threadIdx.x >> 6); w < total; w += gridDim.x * 4) {
    const WaveItem it = wave_item(a, s_cp, nact, rts, w);
    const int row = it.rt * 16 + r16;
    const uint8_t* wr = a.down_q + it.e * mq + (size_t)row * (F / 2);
    const uint16_t* sr = a.down_s + it.e * ms + (size_t)row * G;
    const int ntt = it.n - it.tc > 16 ? 2 : 1;
    int prow[2];  // position of this lane's A-operand row (a real one for absent rows)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) prow[tt] = it.p0 + min(it.tc + 16 * tt + r16, it.n - 1);
    f32x4_t acc[2];
    acc[0] = acc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    DStage s0, s1;
    dn_load<F>(s0, 0, wr, sr, a.h16, prow, q);
    dn_load<F>(s1, min(1, NBLK - 1), wr, sr, a.h16, prow, q);
    for (int b = 0; b < NBLK; b += 2) {
      dn_compute(s0, acc, ntt);
      dn_load<F>(s0, min(b + 2, NBLK - 1), wr, sr, a.h16, prow, q);
      if (b + 1 < NBLK) dn_compute(s1, acc, ntt);
      dn_load<F>(s1, min(b + 3, NBLK - 1), wr, sr, a.h16, prow, q);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt >= ntt) break;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int pt = it.tc + 16 * tt + 4 * q + v;
        if (pt < it.n) a.obuf[(size_t)a.asg[it.p0 + pt] * d + row] = acc[tt][v];
      }
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
  hipLaunchKernelGGL((k_router<D, EPL>), dim3((a.E + 3) / 4, (T + kRouterTokens - 1) / kRouterTokens), dim3(256), 0,
                     s, a, x, r, eps, T, io, wo, xt);
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

// Wave items: (active expert, 16-row tile, 32-token chunk); at most
// min(E, T*k) active experts and T*k/32 extra chunks.
static int grid_for(const LayerArgs& a, int T, int rows) {
  const int Tk = T * a.k;
  const int chunks = (a.E < Tk ? a.E : Tk) + Tk / 32;
  const int wgs = (chunks * (rows / 16) + 3) / 4;
  return wgs < kMaxGroupedGrid ? wgs : kMaxGroupedGrid;
}

hipError_t launch_gateup(const LayerArgs& a, int T, hipStream_t s) {
  const dim3 g(grid_for(a, T, a.f)), b(256);
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
  const dim3 g(grid_for(a, T, a.d)), b(256);
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
