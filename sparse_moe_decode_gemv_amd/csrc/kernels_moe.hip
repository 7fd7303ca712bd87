// kernels_moe.hip -- the decode step of a 4-bit MoE layer for T tokens on gfx950.
//
// Six kernels per call (seven in the stack, whose pre-norm kernel first
// turns the residual into x):
//   router  : logits = W_r x as a matrix product on the matrix cores (x
//             against three exact bf16 terms of W_r), split over K into
//             partial sums.
//   top-k   : one wave per token: the partial sums and bias added in a
//             fixed order, then softmax + top-k; the wave also writes the
//             token's activations in MFMA operand order (fp16), scaled by
//             the power of two 2^a_t that puts their largest magnitude in
//             [1, 2), so any bf16 magnitude converts exactly.
//   sort    : one workgroup of 16 waves: the T*k (token, slot) assignments
//             grouped by expert (a stable counting sort built from wave
//             ballots).
//   gate/up : one workgroup per (chunk of up to 32 tokens of one chosen
//             expert, 64 rows of f): the chunk's activations staged in LDS,
//             int4 weights dequantized into MFMA operands, so each chosen
//             expert's weights are read once per call however many tokens
//             chose it; SwiGLU in registers; h = w_j silu(g) u stored as
//             fp16 operands of the down step.
//   down    : the same over W_d (128 rows of d per workgroup); each
//             assignment's o_{t,j} in fp32.
//   combine : y_t = sum_j o_{t,j} in slot order (deterministic); in the
//             stack the residual add is folded in.
// The pages describe the step: per token a small router picks a few of 256
// routed experts and only those run ("Flint 40B: Best Mid Sized LLM",
// transcript 02:35); kernels for low-bit projections, MoE routing and
// prompt processing are named in the same source (06:11).
//
// MFMA operands.  v_mfma_f32_16x16x32_f16: lane l supplies row l%16 of A
// and column l%16 of B, each with the 8 consecutive k of chunk l/16; lane l
// receives D[4*(l/16)+v][l%16], v = 0..3.  A holds 16 tokens' activations
// (or h), B 16 weight rows, so every lane holds one weight row: the 8 codes
// of one chunk of one group (one stored dword) with that group's scale.
// The lane turns them into fp16 q*s (q = u - 8 exact via the magic number
// 1024, times the scale: one rounding, relative error <= 2^-11), in the
// order e = 0,4,1,5,2,6,3,7 that the magic-number extraction yields (see
// device_common.h); the activation operands are stored in that same order.
// The MFMAs then accumulate over all of K in their C operand.  The
// activations are fp16 here, as x_t 2^a_t (exact, except that elements
// under 2^-14 of the row's largest lose low bits); gate and up then hold
// 2^a_t g and 2^a_t u, SwiGLU stores h 2^(2 a_t) (silu of the true g), and
// the combine scales the token's sum back by 2^(-2 a_t).
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

// One token's 8 activations of one chunk (bf16) times 2^ea as the fp16 MFMA
// operand of the expert kernels, in the order (x0, x4, x1, x5, x2, x6, x3, x7).
__device__ __forceinline__ uint4 operand_chunk(uint4 q, int ea) {
  const float x0 = ldexpf(bf16_bits_to_f32(q.x & 0xFFFFu), ea), x1 = ldexpf(__uint_as_float(q.x & 0xFFFF0000u), ea);
  const float x2 = ldexpf(bf16_bits_to_f32(q.y & 0xFFFFu), ea), x3 = ldexpf(__uint_as_float(q.y & 0xFFFF0000u), ea);
  const float x4 = ldexpf(bf16_bits_to_f32(q.z & 0xFFFFu), ea), x5 = ldexpf(__uint_as_float(q.z & 0xFFFF0000u), ea);
  const float x6 = ldexpf(bf16_bits_to_f32(q.w & 0xFFFFu), ea), x7 = ldexpf(__uint_as_float(q.w & 0xFFFF0000u), ea);
  return make_uint4(pack_f16(x0, x4), pack_f16(x1, x5), pack_f16(x2, x6), pack_f16(x3, x7));
}


// This wave's LDS operations have completed (and act as a compiler barrier).
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Softmax + top-k of one token's E logits in one wave (topk.h): grid T,
// block 64, one token per workgroup (one wave per SIMD of its own: a wave64
// VALU instruction takes 4 cycles, so waves sharing a SIMD would serialize).
// The logits are the S partial sums of the router (slice order) plus the
// bias.
// Token t in one wave; COH: the chosen experts are stored coherently (read
// back by another workgroup of the same kernel).
template <int EPL, int KP, int D, bool COH>
__device__ __forceinline__ void topk_token(const LayerArgs& a, const uint16_t* __restrict__ x, int T, int S,
                                           int32_t* __restrict__ idx_out, float* __restrict__ w_out, int t,
                                           int lane) {
  const int E = a.E, k = a.k, E16 = (E + 15) & ~15;
  // the token's activations, loaded first (they are written back below as
  // the expert kernels' operand row)
  constexpr int XC = D / 8 > 64 ? D / 8 / 64 : 1;  // 8-element chunks per lane
  uint4 xc[XC];
#pragma unroll
  for (int i = 0; i < XC; ++i)
    xc[i] = 64 * i + lane < D / 8 ? reinterpret_cast<const uint4*>(x + (size_t)t * D)[64 * i + lane]
                                  : make_uint4(0u, 0u, 0u, 0u);
  // the router bias (any valid address when there is none: the value is
  // not used), requested with the first partial sums: a conditional load
  // after them would cost one round trip per expert chunk
  const float* bsrc = a.router_b ? a.router_b : a.logits;
  float bv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) bv[i] = bsrc[min(lane + 64 * i, E - 1)];
  constexpr int SU = EPL <= 4 ? 8 : 2;  // slices loaded at a time (all EPL * SU loads in flight)
  const float* p = a.logits + (size_t)t * E16;
  float l[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) l[i] = 0.f;
  for (int s0 = 0; s0 < S; s0 += SU) {
    float q[EPL][SU];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
#pragma unroll
      for (int u = 0; u < SU; ++u) q[i][u] = p[(size_t)min(s0 + u, S - 1) * T * E16 + min(lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
#pragma unroll
      for (int u = 0; u < SU; ++u)
        if (s0 + u < S) l[i] += q[i][u];  // slice order
  }
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const float li = a.router_b ? l[i] + bv[i] : l[i];
    v[i] = lane + 64 * i < E && li == li ? li : -INFINITY;
  }
  int se;
  float sw;
  topk_fast<EPL, KP>(v, E, k, a.norm_topk, lane, se, sw);
  if (lane < k) {
    if constexpr (COH) {
      __hip_atomic_store(a.sel_idx + t * k + lane, se, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      a.sel_idx[t * k + lane] = se;
    }
    a.sel_w[t * k + lane] = sw;
    if (idx_out) idx_out[(size_t)t * k + lane] = se;
    if (w_out) w_out[(size_t)t * k + lane] = sw;
  }
  // operand row: x 2^a with the largest |x| in [1, 2)
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < XC; ++i)
    mb = max(mb, max(max(bf16_mag_max(xc[i].x), bf16_mag_max(xc[i].y)), max(bf16_mag_max(xc[i].z), bf16_mag_max(xc[i].w))));
  const int ea = act_exponent(wave_max_u32(mb));
  uint4* xr = reinterpret_cast<uint4*>(a.xp + (size_t)t * D);
#pragma unroll
  for (int i = 0; i < XC; ++i)
    if (64 * i + lane < D / 8) xr[64 * i + lane] = operand_chunk(xc[i], ea);
  if (lane == 0) a.xexp[t] = ea;
}

template <int EPL, int KP, int D>
__global__ __launch_bounds__(64) void k_topk(const LayerArgs a, const uint16_t* __restrict__ x, int T, int S,
                                             int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  topk_token<EPL, KP, D, false>(a, x, T, S, idx_out, w_out, blockIdx.x, threadIdx.x);
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

// The Tk = T*k assignments a = t*k + j (chosen expert sel[a]) grouped by
// expert, ascending a within an expert:
//   off[e] .. off[e+1]-1  positions of expert e in asg (off[E] = Tk)
//   asg[p]                the assignment at position p
//   act[i], i < meta[0]   the experts with at least one assignment, ascending
//   chunk_off[i]          CS-token chunks of the active experts before act[i]
//                         (chunk_off[meta[0]] = all routed chunks), CS = 32 or 64
//   chunks[c]             chunk c: (expert, first position, positions <= CS)
//   meta[1], meta[2]      all chunks, Tk
// With a shared expert, its T assignments Tk + t sit at positions Tk + t and
// its chunks (expert index E) follow the routed ones.
// Each wave owns a contiguous slice of the assignments: it counts them per
// expert (lanes with equal experts found by wave ballots), a prefix over
// waves gives each (wave, expert) its base, and each wave places its own
// assignments in order: stable, deterministic, no atomics.  Up to 4096
// assignments one workgroup of 16 waves does all of it (k_sort); beyond,
// 64 waves in 16 workgroups count and place, with one workgroup scanning
// between them (k_sort_count, k_sort_scan, k_sort_place).

constexpr int kSortSB = 16;          // chunks of 64 whose expert loads are in flight together
constexpr int kSortWideWaves = 64;   // waves of the three-kernel sort
constexpr int kSortWideMin = 4096;   // assignments from which it is used

template <bool COH>
__device__ __forceinline__ int sel_of(const LayerArgs& a, int i, int E) {
  const int e = COH ? __hip_atomic_load(a.sel_idx + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : a.sel_idx[i];
  return min(max(e, 0), E - 1);
}

// Counts of the wave's slice [a0, a1) into cw[e] (zeroed).
template <bool COH = false>
__device__ void sort_count(const LayerArgs& a, int Tk, int a0, int a1, int lane, int* cw) {
  const int E = a.E;
  for (int cb = a0; cb < a1; cb += 64 * kSortSB) {
    int eb[kSortSB];
#pragma unroll
    for (int u = 0; u < kSortSB; ++u) eb[u] = sel_of<COH>(a, min(cb + 64 * u + lane, Tk - 1), E);
#pragma unroll
    for (int u = 0; u < kSortSB; ++u) {
      const int i = cb + 64 * u + lane;
      if (cb + 64 * u >= a1) break;
      const bool v = i < a1;
      const int e = eb[u];
      const uint64_t same = same_expert_lanes(e, __builtin_amdgcn_ballot_w64(v));
      if (v && lane == __builtin_ctzll(same)) cw[e] += __builtin_popcountll(same);
      lds_wait();
    }
  }
}

// Places the wave's slice: cw[e] holds the next position of expert e.
template <bool COH = false>
__device__ void sort_place(const LayerArgs& a, int Tk, int a0, int a1, int lane, int* cw) {
  const int E = a.E;
  for (int cb = a0; cb < a1; cb += 64 * kSortSB) {
    int eb[kSortSB];
#pragma unroll
    for (int u = 0; u < kSortSB; ++u) eb[u] = sel_of<COH>(a, min(cb + 64 * u + lane, Tk - 1), E);
#pragma unroll
    for (int u = 0; u < kSortSB; ++u) {
      const int i = cb + 64 * u + lane;
      if (cb + 64 * u >= a1) break;
      const bool v = i < a1;
      const int e = eb[u];
      const uint64_t same = same_expert_lanes(e, __builtin_amdgcn_ballot_w64(v));
      const int rank = __builtin_popcountll(same & ((1ull << lane) - 1ull));
      const int pos = v ? cw[e] : 0;
      lds_wait();
      if (v) a.asg[pos + rank] = i;
      if (v && lane == __builtin_ctzll(same)) cw[e] += __builtin_popcountll(same);
      lds_wait();
    }
  }
}

// One wave: from the totals tot[e], the tables off, act, chunk_off, chunks
// and meta; tot[e] becomes the first position of expert e.
__device__ void sort_tables(const LayerArgs& a, int T, int Tk, int CS, int lane, int* tot) {
  const int E = a.E;
  const int pe = (E + 63) / 64;
  const int e0 = min(lane * pe, E), e1 = min(e0 + pe, E);
  int s = 0, na = 0, nc = 0;
  for (int e = e0; e < e1; ++e) {
    const int n = tot[e];
    s += n;
    na += n > 0;
    nc += (n + CS - 1) / CS;
  }
  int base = s, abase = na, cbase = nc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int b1 = __shfl_up(base, o, 64), b2 = __shfl_up(abase, o, 64), b3 = __shfl_up(cbase, o, 64);
    if (lane >= o) {
      base += b1;
      abase += b2;
      cbase += b3;
    }
  }
  base -= s;
  abase -= na;
  cbase -= nc;
  for (int e = e0; e < e1; ++e) {
    const int n = tot[e];
    a.off[e] = base;
    if (n > 0) {
      a.act[abase] = e;
      a.chunk_off[abase] = cbase;
      ++abase;
      for (int tc = 0; tc < n; tc += CS) a.chunks[cbase++] = make_int4(e, base + tc, min(CS, n - tc), 0);
    }
    tot[e] = base;  // from here on: the first position of expert e
    base += n;
  }
  if (lane == 63) {
    a.off[E] = base;
    a.chunk_off[abase] = cbase;
    a.meta[0] = abase;
    // the shared expert (expert index E of the tile-major copies) takes
    // every token, in chunks after the routed ones
    for (int tc = 0; tc < a.ns * T; tc += CS) a.chunks[cbase++] = make_int4(E, Tk + tc, min(CS, T - tc), 0);
    a.meta[1] = cbase;
    a.meta[2] = Tk;
  }
}

// Count and place of a slice that fits one batch (a1 - a0 <= 64 kSortSB),
// from experts the caller loaded once (eb[u]: assignment a0 + 64 u + lane).
__device__ __forceinline__ void batch_count(const int (&eb)[kSortSB], int a0, int a1, int lane, int* cw) {
#pragma unroll
  for (int u = 0; u < kSortSB; ++u) {
    if (a0 + 64 * u >= a1) break;
    const bool v = a0 + 64 * u + lane < a1;
    const uint64_t same = same_expert_lanes(eb[u], __builtin_amdgcn_ballot_w64(v));
    if (v && lane == __builtin_ctzll(same)) cw[eb[u]] += __builtin_popcountll(same);
    lds_wait();
  }
}
__device__ __forceinline__ void batch_place(const LayerArgs& a, const int (&eb)[kSortSB], int a0, int a1, int lane,
                                            int* cw) {
#pragma unroll
  for (int u = 0; u < kSortSB; ++u) {
    const int i = a0 + 64 * u + lane;
    if (a0 + 64 * u >= a1) break;
    const bool v = i < a1;
    const int e = eb[u];
    const uint64_t same = same_expert_lanes(e, __builtin_amdgcn_ballot_w64(v));
    const int rank = __builtin_popcountll(same & ((1ull << lane) - 1ull));
    const int pos = v ? cw[e] : 0;
    lds_wait();
    if (v) a.asg[pos + rank] = i;
    if (v && lane == __builtin_ctzll(same)) cw[e] += __builtin_popcountll(same);
    lds_wait();
  }
}

// The sort in one workgroup of NW waves (up to kSortWideMin assignments).
// LDS: cnt [NW][E], tot [E].  When every wave's slice fits one batch (it
// does for the callers' sizes) the chosen experts are loaded once for the
// count and the placement (one round trip fewer).
template <int NW, bool COH>
__device__ void sort_body(const LayerArgs& a, int T, int CS, int* sm) {
  const int E = a.E, Tk = T * a.k;
  int* cnt = sm;
  int* tot = cnt + NW * E;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int per = (Tk + NW - 1) / NW, a0 = min(wave * per, Tk), a1 = min(a0 + per, Tk);
  const bool one = per <= 64 * kSortSB;
  int eb[kSortSB];
  if (one)
#pragma unroll
    for (int u = 0; u < kSortSB; ++u) eb[u] = sel_of<COH>(a, min(a0 + 64 * u + lane, Tk - 1), E);
  for (int i = tid; i < a.ns * T; i += 64 * NW) a.asg[Tk + i] = Tk + i;  // the shared expert's assignments, last
  for (int i = tid; i < NW * E; i += 64 * NW) cnt[i] = 0;
  __syncthreads();
  int* cw = cnt + wave * E;
  if (one) batch_count(eb, a0, a1, lane, cw);
  else sort_count<COH>(a, Tk, a0, a1, lane, cw);
  __syncthreads();
  for (int e = tid; e < E; e += 64 * NW) {  // base of each wave within expert e, and e's total
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      const int n = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += n;
    }
    tot[e] = run;
  }
  __syncthreads();
  if (wave == 0) sort_tables(a, T, Tk, CS, lane, tot);
  __syncthreads();
  for (int e = lane; e < E; e += 64) cw[e] += tot[e];  // absolute next positions of this wave
  lds_wait();
  if (one) batch_place(a, eb, a0, a1, lane, cw);
  else sort_place<COH>(a, Tk, a0, a1, lane, cw);
}

// One workgroup of 16 waves (up to kSortWideMin assignments).
// LDS (dynamic): cnt [16][E], tot [E].
__global__ __launch_bounds__(1024) void k_sort(const LayerArgs a, int T, int CS) {
  extern __shared__ int sm[];
  sort_body<16, false>(a, T, CS, sm);
}

// Top-k and sort in one kernel (T <= kTopkSortMax): token 4b + w in wave w
// of workgroup b, each wave on a SIMD of its own; the chosen experts are
// stored coherently, every workgroup counts its arrival once they have
// reached the coherence point, and the last to arrive (which resets the
// count) sorts the assignments with its four waves.  LDS: cnt [4][E], tot [E].
constexpr int kTopkSortMax = 128;
template <int EPL, int KP, int D>
__global__ __launch_bounds__(256) void k_topk_sort(const LayerArgs a, const uint16_t* __restrict__ x, int T, int S,
                                                   int32_t* __restrict__ idx_out, float* __restrict__ w_out, int CS) {
  extern __shared__ int sm[];
  __shared__ bool s_last;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t < T) topk_token<EPL, KP, D, true>(a, x, T, S, idx_out, w_out, t, threadIdx.x & 63);
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* ctr = reinterpret_cast<unsigned*>(a.meta + 32);
    s_last = arrive(ctr) == gridDim.x - 1;
    if (s_last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (s_last) sort_body<4, true>(a, T, CS, sm);
}

// Three-kernel sort for many assignments: wave w of kSortWideWaves (16
// workgroups of 4) owns slice w; its counts go to wc[w][E] in the workspace,
// k_sort_scan turns them into per-wave bases and builds the tables, and the
// waves then place their slices.
__global__ __launch_bounds__(256) void k_sort_count(const LayerArgs a, int T) {
  extern __shared__ int sm[];  // [4][E]
  const int E = a.E, Tk = T * a.k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, w = blockIdx.x * 4 + wave;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < a.ns * T; i += gridDim.x * 256) a.asg[Tk + i] = Tk + i;
  int* cw = sm + wave * E;
  for (int e = lane; e < E; e += 64) cw[e] = 0;
  lds_wait();
  const int per = (Tk + kSortWideWaves - 1) / kSortWideWaves, a0 = min(w * per, Tk), a1 = min(a0 + per, Tk);
  sort_count(a, Tk, a0, a1, lane, cw);
  for (int e = lane; e < E; e += 64) a.sort_wc[(size_t)w * E + e] = cw[e];
}

// One workgroup: per expert, the exclusive prefix of the wave counts (the
// wave bases, written back), the totals, then the tables.  LDS: tot [E].
__global__ __launch_bounds__(1024) void k_sort_scan(const LayerArgs a, int T, int CS) {
  extern __shared__ int sm[];
  const int E = a.E, Tk = T * a.k;
  int* tot = sm;
  for (int e = threadIdx.x; e < E; e += 1024) {
    int run = 0;
    for (int w0 = 0; w0 < kSortWideWaves; w0 += 16) {  // 16 loads in flight at a time
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) c[u] = a.sort_wc[(size_t)(w0 + u) * E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        a.sort_wc[(size_t)(w0 + u) * E + e] = run;
        run += c[u];
      }
    }
    tot[e] = run;
  }
  __syncthreads();
  if (threadIdx.x < 64) sort_tables(a, T, Tk, CS, threadIdx.x, tot);
}

__global__ __launch_bounds__(256) void k_sort_place(const LayerArgs a, int T) {
  extern __shared__ int sm[];  // [4][E]
  const int E = a.E, Tk = T * a.k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, w = blockIdx.x * 4 + wave;
  int* cw = sm + wave * E;
  for (int e = lane; e < E; e += 64) cw[e] = a.off[e] + a.sort_wc[(size_t)w * E + e];
  lds_wait();
  const int per = (Tk + kSortWideWaves - 1) / kSortWideWaves, a0 = min(w * per, Tk), a1 = min(a0 + per, Tk);
  sort_place(a, Tk, a0, a1, lane, cw);
}

// Tokens per chunk of the expert kernels: 64 once the experts average 32
// or more assignments (each weight dequantized once per 64 tokens), else 32.
int chunk_rows(const LayerArgs& a, int T) { return (long long)T * a.k >= 32LL * a.E ? 64 : 32; }

size_t sort_lds_bytes(int E, int Tk) {
  (void)Tk;
  return (size_t)(17 * E) * sizeof(int);
}

// ----------------------------------------------------------------- router

// Router logits of T tokens as one matrix product on the matrix cores:
// logits[t][e] = sum_k x[t][k] W_r[e][k].  The fp32 router matrix is held
// (from init) as three bfloat16 terms per weight, w = h + m + l exactly
// (each term takes the next 8 significant bits of what the previous ones
// left; exact for |w| >= 2^-100), so the three bf16 MFMAs per tile form
// every product x * w exactly in fp32 and the only rounding is the fp32
// accumulation, as in an fp32 dot product.  A workgroup computes 64 experts
// (16 per wave) x 16*NB tokens over one slice of K (split K: enough
// workgroups to fill the chip at any T); each slice's sums go to its own
// partial array and the top-k kernel adds the slices and the bias in a
// fixed order, so the result does not depend on timing.
constexpr int kRtE = 64;       // experts per workgroup
constexpr int kRtGrid = 256;   // workgroups aimed for (one per CU)
constexpr int kRtMinK = 128;   // smallest K slice of one workgroup
constexpr int kRtRow = 5;      // uint4 per staged token row: 4 of x (32 bf16) + 1 of padding

// 16-token blocks per workgroup: up to 8 (128 tokens), fewer for small T.
int router_nb(int T) { return T <= 16 ? 1 : T <= 32 ? 2 : T <= 64 ? 4 : 8; }

int router_splits(int T, int E, int d) {
  const int tt = 16 * router_nb(T);
  const int tiles = ((T + tt - 1) / tt) * ((E + kRtE - 1) / kRtE);
  int S = 1;
  while (2 * S * tiles <= kRtGrid && 2 * S <= d / kRtMinK) S *= 2;
  return S;
}

size_t router_partial_floats(int T, int E, int d) {
  return (size_t)router_splits(T, E, d) * T * ((E + 15) & ~15);
}

// One thread per (16-row block eb, 32-column block kb, lane l): the weights
// W_r[16eb + l%16][32kb + 8(l/16) + i], i = 0..7 (zero past row E), as their
// three bf16 terms, stored as tiles [eb][kb][term][64 lanes] of uint4 (the
// MFMA A-operand of lane l).
__global__ __launch_bounds__(256) void k_router_terms(const float* __restrict__ w, int E, int d,
                                                      uint4* __restrict__ out) {
  const int nkb = d / 32;
  const size_t n = (size_t)((E + 15) / 16) * nkb * 64;
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= n) return;
  const int l = (int)(g & 63);
  const size_t tile = g >> 6;
  const int kb = (int)(tile % nkb), eb = (int)(tile / nkb);
  const int e = eb * 16 + (l & 15), k0 = kb * 32 + 8 * (l >> 4);
  float v[8];
  const float4* src = reinterpret_cast<const float4*>(w + (size_t)min(e, E - 1) * d + k0);
  const float4 v0 = src[0], v1 = src[1];
  v[0] = v0.x, v[1] = v0.y, v[2] = v0.z, v[3] = v0.w, v[4] = v1.x, v[5] = v1.y, v[6] = v1.z, v[7] = v1.w;
  uint32_t th[4], tm[4], tl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = e < E ? v[2 * j] : 0.f, b = e < E ? v[2 * j + 1] : 0.f;
    th[j] = pack_bf16(a, b);
    const float ra = a - bf16_bits_to_f32(th[j] & 0xFFFFu), rb = b - __uint_as_float(th[j] & 0xFFFF0000u);
    tm[j] = pack_bf16(ra, rb);
    const float sa = ra - bf16_bits_to_f32(tm[j] & 0xFFFFu), sb = rb - __uint_as_float(tm[j] & 0xFFFF0000u);
    tl[j] = pack_bf16(sa, sb);
  }
  out[(tile * 3 + 0) * 64 + l] = make_uint4(th[0], th[1], th[2], th[3]);
  out[(tile * 3 + 1) * 64 + l] = make_uint4(tm[0], tm[1], tm[2], tm[3]);
  out[(tile * 3 + 2) * 64 + l] = make_uint4(tl[0], tl[1], tl[2], tl[3]);
}

// Pre-norm of the stack: x_t = bf16(r_t / sqrt(mean(r_t^2) + eps)), one wave
// per token.
template <int D>
__global__ __launch_bounds__(64) void k_prenorm(const float* __restrict__ resid, float eps,
                                                uint16_t* __restrict__ xn) {
  constexpr int NI = D / 256;  // float4 per lane: columns 4*lane + 256*i
  const int t = blockIdx.x, lane = threadIdx.x;
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
  uint2* xr = reinterpret_cast<uint2*>(xn + (size_t)t * D);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    xr[64 * i + lane] = make_uint2(pack_bf16(rv[i].x / den, rv[i].y / den), pack_bf16(rv[i].z / den, rv[i].w / den));
}


// grid = ceil(E/64) * ceil(T/(16 NB)) * S workgroups of 256.  Wave w holds
// the A operands (16 experts x 32 k, three terms) of its expert block; the
// workgroup stages its 16 NB tokens' x (32 k per step) in LDS, double
// buffered, and each wave reads its B operands (16 tokens x 32 k) there.
// Rows past T hold token T-1 again (loads clamped); their sums are not
// stored.  Lane l ends with the logits of token 16j + l%16, experts
// 4(l/16) .. +3 of its block.
template <int NB>
__global__ __launch_bounds__(256) void k_router_mm(const LayerArgs a, const uint16_t* __restrict__ x, int T,
                                                   int S) {
  constexpr int TT = 16 * NB;                  // tokens per workgroup
  constexpr int NC = (4 * TT + 255) / 256;     // staged 16-byte chunks per thread and step
  __shared__ uint4 s_x[2][TT * kRtRow];
  const int d = a.d, E16 = (a.E + 15) & ~15, nkb = d / 32;
  const int NET = (a.E + kRtE - 1) / kRtE, NTT = (T + TT - 1) / TT;
  // consecutive work items on one XCD (blocks go round-robin over the 8 XCDs)
  const int N = gridDim.x, bi = blockIdx.x;
  const int w = (N & 7) == 0 ? (bi & 7) * (N >> 3) + (bi >> 3) : bi;
  const int et = w % NET, tt = (w / NET) % NTT, sk = w / (NET * NTT);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool eb_ok = et * 4 + wave < E16 / 16;
  const int eb = min(et * 4 + wave, E16 / 16 - 1);
  const int nk = nkb / S, kb0 = sk * nk;
  const int t0 = tt * TT;

  const uint4* wa = reinterpret_cast<const uint4*>(a.router_t) + ((size_t)eb * nkb + kb0) * 192 + lane;
  // staging: chunk c = threadIdx.x + 256 i is chunk c%4 of token row c/4
  const bool st_ok = 4 * TT >= 256 || (int)threadIdx.x < 4 * TT;
  const uint4* xs[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = threadIdx.x + 256 * i, t = t0 + c / 4;
    xs[i] = reinterpret_cast<const uint4*>(x + (size_t)min(t, T - 1) * d + kb0 * 32) + (c & 3);
  }

  // operands of 4 steps in flight (a ring of register slots; nk is a
  // multiple of 4): step ks + 4 is loaded into the slot step ks has used.
  // Past the end the loads repeat the last step (unconditional loads).
  uint4 Ar[4][3], Xr[4][NC];
  auto load = [&](uint4 (&A)[3], uint4 (&X)[NC], int ks) {
#pragma unroll
    for (int i = 0; i < NC; ++i) X[i] = xs[i][ks * 4];
#pragma unroll
    for (int p = 0; p < 3; ++p) A[p] = wa[(size_t)ks * 192 + p * 64];
  };
  auto stage = [&](int buf, const uint4 (&X)[NC], int ks) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = threadIdx.x + 256 * i;
      if (st_ok) s_x[buf][(c >> 2) * kRtRow + (c & 3)] = X[i];
    }
  };
#pragma unroll
  for (int u = 0; u < 4; ++u) load(Ar[u], Xr[u], u);
  stage(0, Xr[0], 0);
  __syncthreads();

  f32x4_t acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int ks0 = 0; ks0 < nk; ks0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ks = ks0 + u;
      const uint4* sb = s_x[u & 1];
      uint4 B[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) B[j] = sb[(16 * j + (lane & 15)) * kRtRow + (lane >> 4)];
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Ar[u][p]),
                                                           __builtin_bit_cast(bf16x8_t, B[j]), acc[j], 0, 0, 0);
      // the next step's x into the other buffer (the last step restages its own)
      stage((u + 1) & 1, Xr[(u + 1) & 3], min(ks + 1, nk - 1));
      __syncthreads();
      load(Ar[u], Xr[u], min(ks + 4, nk - 1));
    }
  }

  if (eb_ok) {
    float* part = a.logits + (size_t)sk * T * E16 + eb * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = t0 + 16 * j + (lane & 15);
      if (t < T) {
        const f32x4_t v = acc[j];
        *reinterpret_cast<float4*>(part + (size_t)t * E16) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

// ----------------------------------------------------------------- MFMA tiles

__device__ __forceinline__ uint32_t dword_of(uint4 v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }

// 0x64006400 held in a VGPR the compiler cannot see into, so that each
// (mask, magic) pair is one 3-input bitwise instruction (a VALU instruction
// takes at most one literal).
__device__ __forceinline__ uint32_t magic_f16x2() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

// B operand of one MFMA: the 8 codes of one dword as fp16 q * s, with s2
// the group's binary16 scale in both halves and magic = 0x64006400.
__device__ __forceinline__ f16x8_t dequant_f16(uint32_t w, f16x2_t s2, uint32_t magic) {
  const f16x2_t off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2_t sx = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2_t so = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w8 = w >> 8;
  // exact q: (1024+u) - 1032 for even e, (1024+16u)/16 - 72 for odd e
  const f16x2_t q0 = __builtin_bit_cast(f16x2_t, (w & 0x000F000Fu) | magic) + off;
  const f16x2_t q1 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, (w & 0x00F000F0u) | magic), sx, so);
  const f16x2_t q2 = __builtin_bit_cast(f16x2_t, (w8 & 0x000F000Fu) | magic) + off;
  const f16x2_t q3 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, (w8 & 0x00F000F0u) | magic), sx, so);
  const uint4 v = make_uint4(__builtin_bit_cast(uint32_t, q0 * s2), __builtin_bit_cast(uint32_t, q1 * s2),
                             __builtin_bit_cast(uint32_t, q2 * s2), __builtin_bit_cast(uint32_t, q3 * s2));
  return __builtin_bit_cast(f16x8_t, v);
}

// scale j (0..3) of the four binary16 scales in sc, in both halves
__device__ __forceinline__ f16x2_t scale2(uint2 sc, int j) {
  const uint32_t d = (j & 2) ? sc.y : sc.x;
  return __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(d, d, (j & 1) ? 0x03020302u : 0x01000100u));
}

// ----------------------------------------------------------------- grouped items

// Work item of one workgroup: (chunk of up to 32 or 64 positions of one
// expert, group of weight rows).  The chunk list (grouped by expert) is cut
// into 8 contiguous ranges, one per XCD (workgroups go round-robin over the
// 8 XCDs, and the grid is a multiple of 8), so the row groups of a chunk
// share one L2 for its activations, and the chunks of an expert share it
// for the weights (but at the 7 cuts).  Within an XCD, item i is chunk
// i / ngroups of the range, row group i % ngroups.  The chunk table is read
// directly (one round trip from the start of the kernel to the operand
// loads' addresses).
struct Item {
  int e, rg, p0, n;
};
struct ItemRange {
  int c0, n, step;  // first chunk, items, item stride of this workgroup
};
__device__ __forceinline__ ItemRange xcd_items(const LayerArgs& a, int ngroups) {
  const int C = a.meta[1], x = blockIdx.x & 7;
  const int c0 = x * C / 8, c1 = (x + 1) * C / 8;
  return ItemRange{c0, (c1 - c0) * ngroups, (int)gridDim.x >> 3};
}
__device__ __forceinline__ Item item_of(const LayerArgs& a, const ItemRange& r, int ngroups, int i) {
  const int c = i / ngroups;
  const int4 cd = a.chunks[r.c0 + c];
  Item it;
  it.e = cd.x;
  it.p0 = cd.y;
  it.n = cd.z;
  it.rg = i - c * ngroups;
  return it;
}

// Small T (32-token chunks, about one per chosen expert) takes another
// order: chunk c goes to XCD c % 8 with all its row groups (which share
// the chunk's activation or h rows in that XCD's L2), and workgroup slot j
// (blockIdx / 8) of the XCD takes its items j, j + S, j + 2S, ... (S =
// gridDim / 8), item i being chunk x + 8 (i / ngroups), row group i %
// ngroups.  The first item's chunk is known before the chunk count, so its
// table entry is requested together with the count: one round trip before
// the item's own loads instead of two.  (Large T keeps the contiguous
// ranges above, where consecutive chunks of one expert share the L2 for
// its weights.)
struct ItemWalk {
  int x, j0, S, C, ngroups, cap;
  int4 first;  // the table entry of the first item (clamped into the table)
};
__device__ __forceinline__ ItemWalk walk_start(const LayerArgs& a, int ngroups) {
  ItemWalk w;
  w.x = blockIdx.x & 7, w.j0 = blockIdx.x >> 3, w.S = gridDim.x >> 3, w.ngroups = ngroups, w.cap = a.chunk_cap;
  w.first = a.chunks[min(w.x + 8 * (w.j0 / ngroups), w.cap - 1)];
  w.C = a.meta[1];
  asm volatile("" ::: "memory");  // both reads issued here, not sunk to their uses
  return w;
}
// Item i of the walk; false past the last chunk.
__device__ __forceinline__ bool walk_item(const LayerArgs& a, const ItemWalk& w, int i, Item& it) {
  const int c = w.x + 8 * (i / w.ngroups);
  if (c >= w.C) return false;
  const int4 cd = i == w.j0 ? w.first : a.chunks[c];
  it.e = cd.x;
  it.p0 = cd.y;
  it.n = cd.z;
  it.rg = i - (i / w.ngroups) * w.ngroups;
  return true;
}

// The operand rows of one 128-element block of K for the item's (up to)
// 16*NTT rows (tokens or positions), in LDS in fragment order:
// v[tt][j][q][slot] is chunk q of group j of row 16*tt + r, at slot
// r ^ swz(j, q), so that the 64 lanes of a wave read one (tt, j) as 1 KB
// with every 16 lanes covering all banks, and the staging stores (8 rows x
// 8 parts per wave) hit distinct banks too.
template <int NTT>
struct OpTile {
  uint4 v[NTT][4][4][16];
};
__device__ __forceinline__ int swz(int j, int q) { return (4 * j + 2 * (q >> 1)) & 15; }

// Thread i stages 32 bytes (16 elements: group p/2, chunks 2(p%2) and
// 2(p%2)+1) of row c = i/8 + 32 m, part p = i%8, for each pass m < NTT/2.
template <int NP>
struct StageRegs {
  uint4 a[NP], b[NP];
};
template <int NP>
__device__ __forceinline__ StageRegs<NP> stage_load(int blk, const uint16_t* const (&rows)[NP], int tid) {
  StageRegs<NP> r;
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    const uint4* src = reinterpret_cast<const uint4*>(rows[m] + blk * 128 + 16 * (tid & 7));
    r.a[m] = src[0];
    r.b[m] = src[1];
  }
  return r;
}
template <int NTT>
__device__ __forceinline__ void stage_store(OpTile<NTT>& t, const StageRegs<NTT / 2>& r, int tid) {
  const int p = tid & 7, j = p >> 1, q0 = 2 * (p & 1);
#pragma unroll
  for (int m = 0; m < NTT / 2; ++m) {
    const int c = (tid >> 3) + 32 * m, r16 = c & 15;
    t.v[c >> 4][j][q0][r16 ^ swz(j, q0)] = r.a[m];
    t.v[c >> 4][j][q0 + 1][r16 ^ swz(j, q0 + 1)] = r.b[m];
  }
}

// Tile-major copy of an expert matrix [R rows][K] (made once at init for
// the batched step): unit (tile of 16 rows, block of 128 k) holds, at
// 16-byte word 16*q + r, piece q of that block of row 16*tile + r -- the
// lane order of an MFMA operand -- so one wave load reads 1 KB contiguous
// and a tile streams sequentially; its scales sit at 8-byte word r of a
// 128-byte unit (the block's 4 group scales of row r).
__global__ __launch_bounds__(256) void k_tile_codes(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                    long long rows, int K) {
  const int ppr = K / 32;  // pieces per row
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * ppr) return;
  const long long row = i / ppr;
  const int c = (int)(i - row * ppr), kb = c >> 2, q = c & 3;
  const long long tile = row >> 4;
  dst[(tile * (K / 128) + kb) * 64 + q * 16 + (row & 15)] = src[i];
}
// U: one row's 4 scales of a 128-element block (uint2: binary16, int4;
// uint32_t: E8M0 bytes, MXFP4)
template <typename U>
__global__ __launch_bounds__(256) void k_tile_scales(const U* __restrict__ src, U* __restrict__ dst,
                                                     long long rows, int K) {
  const int upr = K / 128;  // 4-scale units per row
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * upr) return;
  const long long row = i / upr;
  const int kb = (int)(i - row * upr);
  dst[((row >> 4) * upr + kb) * 16 + (row & 15)] = src[i];
}

// NVFP4 scales into the tile-major order with the matrix scale folded in:
// thread (row, block kb, half h) writes the fp16 values of the row's E4M3
// scales h, h+2, h+4, h+6 of that 128-element block times the row's matrix
// scale (rounded once to fp16) -- the 4 scales a lane of piece q, h = q/2,
// uses -- at unit ((row/16) * K/128 + kb) * 32 + 16 h + row % 16.
__global__ __launch_bounds__(256) void k_tile_scales_nv(const uint8_t* __restrict__ src, const float* __restrict__ tsc,
                                                        long long rows_per_mat, long long rows, int K,
                                                        uint2* __restrict__ dst) {
  const int upr = K / 128;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * upr * 2) return;
  const int h = (int)(i & 1);
  const long long ru = i >> 1, row = ru / upr;
  const int kb = (int)(ru - row * upr);
  const uint2 b = *reinterpret_cast<const uint2*>(src + row * (K / 16) + 8 * kb);
  const float t = tsc[row / rows_per_mat];
  uint32_t f[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bi = 2 * j + h;
    const uint32_t byte = ((bi < 4 ? b.x : b.y) >> (8 * (bi & 3))) & 0xFFu;
    f[j] = __builtin_bit_cast(uint16_t, (_Float16)(e4m3_f32(byte) * t));
  }
  dst[((row >> 4) * upr + kb) * 32 + 16 * h + (row & 15)] = make_uint2(f[0] | (f[1] << 16), f[2] | (f[3] << 16));
}

// Weights of one block for one 16-row tile: this lane's row, chunk q of the
// block's 4 groups, and the 4 group scales, from the tile-major copy.
struct WBlk {
  uint4 q;
  uint2 s;
};
// FMT: 0 int4 (4 binary16 scales per row and block: 8 bytes), 1 MXFP4 (4
// E8M0 bytes), 2 NVFP4 (per row and block two sets of 4 fp16 scales, the
// matrix scale folded in; a lane takes the set of its piece's half)
template <int FMT>
__device__ __forceinline__ WBlk wload(const uint4* tq, const uint2* ts, int blk, int lane) {
  WBlk w;
  w.q = tq[blk * 64 + lane];
  if constexpr (FMT == 1) w.s = make_uint2(reinterpret_cast<const uint32_t*>(ts)[blk * 16 + (lane & 15)], 0u);
  else if constexpr (FMT == 2) w.s = ts[blk * 32 + 16 * (lane >> 5) + (lane & 15)];
  else w.s = ts[blk * 16 + (lane & 15)];
  return w;
}

// Scales of tile unit `off` (units of one row's block scales: 16 per tile
// and block) of a tile-major scale copy.
template <int FMT>
__device__ __forceinline__ const uint2* tile_scales(const uint16_t* base, size_t off) {
  if constexpr (FMT == 1) return reinterpret_cast<const uint2*>(reinterpret_cast<const uint32_t*>(base) + off);
  else if constexpr (FMT == 2) return reinterpret_cast<const uint2*>(base) + 2 * off;
  else return reinterpret_cast<const uint2*>(base) + off;
}

// FP4 B operand of one MFMA: the 8 E2M1 codes of one dword times `scale`,
// a power of two (the conversion's scale operand is an MX block scale: only
// its exponent counts; exact for E8M0 bytes 104..140), as fp16 (one
// v_cvt_scalef32_pk_f16_fp4 per code pair), reordered into the int4
// operand order (e0,e4), (e1,e5), (e2,e6), (e3,e7) that the activation rows
// use.
template <int B>
__device__ __forceinline__ uint32_t fp4_pair_f16s(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, B));
}
__device__ __forceinline__ f16x8_t dequant_fp4_f16(uint32_t w, float scale) {
  const uint32_t p01 = fp4_pair_f16s<0>(w, scale), p23 = fp4_pair_f16s<1>(w, scale);
  const uint32_t p45 = fp4_pair_f16s<2>(w, scale), p67 = fp4_pair_f16s<3>(w, scale);
  const uint4 v = make_uint4(__builtin_amdgcn_perm(p45, p01, 0x05040100u), __builtin_amdgcn_perm(p45, p01, 0x07060302u),
                             __builtin_amdgcn_perm(p67, p23, 0x05040100u), __builtin_amdgcn_perm(p67, p23, 0x07060302u));
  return __builtin_bit_cast(f16x8_t, v);
}

// One block of K for two weight tiles against the NTT staged token tiles:
// each weight dword is dequantized once and used by NTT MFMAs.
// NVFP4 B operand: the codes converted exactly (scale 1), then one fp16
// multiply by s2, the block's E4M3 value times the matrix scale (rounded to
// fp16 once, at init): two roundings of 2^-11, like int4's q * s.
__device__ __forceinline__ f16x8_t dequant_nv_f16(uint32_t w, f16x2_t s2) {
  const f16x8_t s8 = {s2.x, s2.y, s2.x, s2.y, s2.x, s2.y, s2.x, s2.y};
  return dequant_fp4_f16(w, 1.0f) * s8;
}

template <int NTT, int FMT>
__device__ __forceinline__ void block_mfma(f32x4_t (&acc)[2][NTT], const OpTile<NTT>& t, const WBlk (&w)[2],
                                           int lane, uint32_t magic) {
  const int q = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f16x8_t wb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (FMT == 2) {
        // dword j of piece q spans elements 32j + 8q .. +7: 16-block 2j + q/2,
        // scale j of the lane's set
        wb[i] = dequant_nv_f16(dword_of(w[i].q, j), scale2(w[i].s, j));
      } else if constexpr (FMT == 1) {
        wb[i] = dequant_fp4_f16(dword_of(w[i].q, j), ldexpf(1.0f, (int)((w[i].s.x >> (8 * j)) & 0xFFu) - 127));
      } else {
        wb[i] = dequant_f16(dword_of(w[i].q, j), scale2(w[i].s, j), magic);
      }
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const f16x8_t xa = __builtin_bit_cast(f16x8_t, t.v[tt][j][q][r16 ^ swz(j, q)]);
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, wb[i], acc[i][tt], 0, 0, 0);
    }
  }
}

// The K loop shared by both kernels: NBLK blocks; the operand tile is
// double-buffered in LDS (one barrier per block) and fed from a ring of up
// to 4 blocks of staging loads in registers.  Each wave's two weight tiles
// come in groups of G = 2 consecutive blocks (2 KB of the tile-major copy
// each), double-buffered: the loads of group g+1 are issued when group g
// starts.  (4 + 2 measured 3 % faster than 2 + 4 at T = 64, equal at
// T = 2048.)  Every global load is unconditional (rows past the chunk
// are clamped to a real one and their outputs dropped), so the compiler's
// wait counts stay exact.
template <int K>
constexpr int kloop_g() { return K / 128 < 2 ? K / 128 : 2; }  // weight blocks per burst

// The first burst of the two weight tiles, requested by the caller as soon
// as the item is known (the weights depend only on the expert and the row
// group, not on the tokens).
template <int K, int FMT>
__device__ __forceinline__ void k_loop_first(WBlk (&w0)[kloop_g<K>()][2], const uint4* const (&wtq)[2],
                                             const uint2* const (&wts)[2], int lane) {
#pragma unroll
  for (int i = 0; i < kloop_g<K>(); ++i)
#pragma unroll
    for (int m = 0; m < 2; ++m) w0[i][m] = wload<FMT>(wtq[m], wts[m], i, lane);
}

template <int K, int NTT, int FMT>
__device__ __forceinline__ void k_loop(f32x4_t (&acc)[2][NTT], OpTile<NTT>* tiles,
                                       const uint16_t* const (&op_rows)[NTT / 2], const uint4* const (&wtq)[2],
                                       const uint2* const (&wts)[2], WBlk (&w)[2][kloop_g<K>()][2], int tid,
                                       int lane, uint32_t magic) {
  constexpr int NBLK = K / 128;
  constexpr int G = kloop_g<K>();           // weight blocks per burst (w[0]: requested by the caller)
  constexpr int SX = NBLK < 4 ? NBLK : 4;   // operand blocks in flight
  StageRegs<NTT / 2> sx[SX];
#pragma unroll
  for (int i = 0; i < SX; ++i) sx[i] = stage_load(i, op_rows, tid);
  stage_store(tiles[0], sx[0], tid);
  sx[0] = stage_load(min(SX, NBLK - 1), op_rows, tid);
  __syncthreads();
  for (int b0 = 0; b0 < NBLK; b0 += 2 * G) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g0 = b0 + h * G;  // first block of this group
      if (NBLK > G) {
        // the next group's burst (clamped past the end: repeats the last group)
        const int n0 = min(g0 + G, NBLK - G);
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
          for (int m = 0; m < 2; ++m) w[h ^ 1][i][m] = wload<FMT>(wtq[m], wts[m], n0 + i, lane);
      }
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int b = g0 + i;
        if (b < NBLK) {
          block_mfma<NTT, FMT>(acc, tiles[b & 1], w[h][i], lane, magic);
          // slot (b+1) % SX holds block b+1: into the other LDS buffer, then refill
          stage_store(tiles[(b + 1) & 1], sx[(b + 1) % SX], tid);
          sx[(b + 1) % SX] = stage_load(min(b + 1 + SX, NBLK - 1), op_rows, tid);
          __syncthreads();
        }
      }
    }
  }
}

// ----------------------------------------------------------------- gate/up

// Item: (chosen expert, 64 rows of f, up to 16*NTT tokens).  Wave w takes
// gate and up rows 16w .. 16w+15 of the group; K = d.  Epilogue in
// registers: h = w_j * silu(g) * u, written as fp16 in operand order
// (0,4,1,5,2,6,3,7 within each 8 rows) for the down step.
template <int D, int NTT, int FMT>
__global__ __launch_bounds__(256, 2) void k_gateup(const LayerArgs a) {
  __shared__ OpTile<NTT> s_tile[2];
  const int f = a.f, k = a.k, ngroups = f / 64;
  constexpr bool WALK = NTT == 2;  // 32-token chunks: the small-T order (walk_item)
  ItemRange ir{};
  ItemWalk wk{};
  if constexpr (WALK) wk = walk_start(a, ngroups);
  else ir = xcd_items(a, ngroups);
  const uint32_t magic = magic_f16x2();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, q = lane >> 4;
  for (int i = blockIdx.x >> 3;; i += WALK ? wk.S : ir.step) {
    Item it;
    if constexpr (WALK) {
      if (!walk_item(a, wk, i, it)) break;
    } else {
      if (i >= ir.n) break;
      it = item_of(a, ir, ngroups, i);
    }
    const size_t tile = (size_t)it.e * (f / 16) + it.rg * 4 + wave;  // 16-row tile of gate and of up
    const uint4* wtq[2] = {reinterpret_cast<const uint4*>(a.gate_t) + tile * (D / 128) * 64,
                           reinterpret_cast<const uint4*>(a.up_t) + tile * (D / 128) * 64};
    const uint2* wts[2] = {tile_scales<FMT>(a.gate_ts, tile * (D / 128) * 16),
                           tile_scales<FMT>(a.up_ts, tile * (D / 128) * 16)};

    // The item's assignments are requested first: those of the operand
    // rows this thread stages (chunk rows tid/8 + 32m) and those of this
    // lane's output tokens (4q+v of each tile; rows past the chunk repeat
    // its last assignment).  Then the first weight burst, which needs only
    // the expert, so it is in flight while the rows' addresses come back;
    // the epilogue's per-token values (slot weight, activation exponent)
    // are fetched while the K loop runs.
    const int Tk = a.meta[2];
    int asg_r[NTT / 2], asg_o[NTT][4];
#pragma unroll
    for (int m = 0; m < NTT / 2; ++m) asg_r[m] = a.asg[it.p0 + min((tid >> 3) + 32 * m, it.n - 1)];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) asg_o[tt][v] = a.asg[it.p0 + min(16 * tt + 4 * q + v, it.n - 1)];
    WBlk w[2][kloop_g<D>()][2];
    k_loop_first<D, FMT>(w[0], wtq, wts, lane);
    const uint16_t* rows[NTT / 2];
#pragma unroll
    for (int m = 0; m < NTT / 2; ++m) {
      const int tok = asg_r[m] < Tk ? asg_r[m] / k : asg_r[m] - Tk;  // shared-expert assignments: Tk + token
      rows[m] = a.xp + (size_t)tok * D;
    }
    float wjv[NTT][4];
    int eav[NTT][4];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int asg = asg_o[tt][v];
        wjv[tt][v] = asg < Tk ? a.sel_w[asg] : 1.f;
        eav[tt][v] = a.xexp[asg < Tk ? asg / k : asg - Tk];
      }
    f32x4_t acc[2][NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[0][tt] = acc[1][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // all token tiles always (rows past the chunk repeat a real row and
    // their outputs are dropped): one code path
    k_loop<D, NTT, FMT>(acc, s_tile, rows, wtq, wts, w, tid, lane, magic);
    // lane: weight row r16, tokens 4q+v of each tile
    const int e8 = r16 & 7;
    const int col = it.rg * 64 + wave * 16 + (r16 & 8) + 2 * (e8 & 3) + (e8 >> 2);  // h in operand order
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      if (16 * tt >= it.n) break;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int pt = 16 * tt + 4 * q + v;
        if (pt < it.n) {
          // gate and up hold 2^ea g and 2^ea u: h 2^(2 ea) with silu of the true g
          const float gs = acc[0][tt][v];
          const float h = wjv[tt][v] * (gs / (1.0f + expf(-ldexpf(gs, -eav[tt][v])))) * acc[1][tt][v];
          a.h16[(size_t)(it.p0 + pt) * f + col] = __builtin_bit_cast(uint16_t, (_Float16)h);
        }
      }
    }
  }
}

// ----------------------------------------------------------------- down

// Item: (chosen expert, 128 rows of d, up to 16*NTT tokens).  Wave w takes
// rows 32w .. 32w+31 of the group as two tiles; K = f, against the fp16 h
// operands.  o_{t,j} goes to obuf[t*k + j][row].
template <int F, int NTT, int FMT>
__global__ __launch_bounds__(256, 2) void k_down(const LayerArgs a) {
  __shared__ OpTile<NTT> s_tile[2];
  const int d = a.d, ngroups = d / 128;
  constexpr bool WALK = NTT == 2;  // 32-token chunks: the small-T order (walk_item)
  ItemRange ir{};
  ItemWalk wk{};
  if constexpr (WALK) wk = walk_start(a, ngroups);
  else ir = xcd_items(a, ngroups);
  const uint32_t magic = magic_f16x2();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, q = lane >> 4;
  for (int i = blockIdx.x >> 3;; i += WALK ? wk.S : ir.step) {
    Item it;
    if constexpr (WALK) {
      if (!walk_item(a, wk, i, it)) break;
    } else {
      if (i >= ir.n) break;
      it = item_of(a, ir, ngroups, i);
    }
    const int row0 = it.rg * 128 + wave * 32 + r16;
    const size_t tile = (size_t)it.e * (d / 16) + it.rg * 8 + wave * 2;  // two 16-row tiles of W_d
    const uint4* wtq[2] = {reinterpret_cast<const uint4*>(a.down_t) + tile * (F / 128) * 64,
                           reinterpret_cast<const uint4*>(a.down_t) + (tile + 1) * (F / 128) * 64};
    const uint2* wts[2] = {tile_scales<FMT>(a.down_ts, tile * (F / 128) * 16),
                           tile_scales<FMT>(a.down_ts, (tile + 1) * (F / 128) * 16)};

    const uint16_t* rows[NTT / 2];
#pragma unroll
    for (int m = 0; m < NTT / 2; ++m) rows[m] = a.h16 + (size_t)(it.p0 + min((tid >> 3) + 32 * m, it.n - 1)) * F;
    // the assignments this lane's outputs go to, fetched while the K loop runs
    int dst[NTT][4];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[tt][v] = a.asg[it.p0 + min(16 * tt + 4 * q + v, it.n - 1)];
    f32x4_t acc[2][NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[0][tt] = acc[1][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    WBlk w[2][kloop_g<F>()][2];
    k_loop_first<F, FMT>(w[0], wtq, wts, lane);
    k_loop<F, NTT, FMT>(acc, s_tile, rows, wtq, wts, w, tid, lane, magic);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      if (16 * tt >= it.n) break;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int pt = 16 * tt + 4 * q + v;
        if (pt < it.n) {
          float* o = a.obuf + (size_t)dst[tt][v] * d + row0;
          o[0] = acc[0][tt][v];
          o[16] = acc[1][tt][v];
        }
      }
    }
  }
}

// ----------------------------------------------------------------- combine

// y_t = 2^(-2 a_t) sum_{j<k} o_{t,j} (slot order); with resid, resid_t += y_t.
// KP: k rounded up to a power of two.  Every row of the sum, the shared
// expert's, the exponent and the residual are requested before any is used
// (rows past k, and the shared row without a shared expert, repeat a real
// row and are not added), so the thread waits one round trip, not one per
// slot.
template <int KP>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ obuf, const int32_t* __restrict__ xexp,
                                                 int T, int d, int k, int ns, float* __restrict__ y_out,
                                                 float* __restrict__ resid) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // float4 index over [T][d]
  if (i >= T * d / 4) return;
  const int t = (4 * i) / d, r = 4 * i - t * d;
  float4 o[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) o[j] = *reinterpret_cast<const float4*>(obuf + ((size_t)t * k + min(j, k - 1)) * d + r);
  const float4 osh = *reinterpret_cast<const float4*>(obuf + (ns ? (size_t)T * k + t : (size_t)t * k) * d + r);
  const int ea = xexp[t];
  float4* rp = reinterpret_cast<float4*>((resid ? resid : y_out) + (size_t)t * d + r);
  const float4 rv0 = resid ? *rp : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    if (j < k) {
      s.x += o[j].x;
      s.y += o[j].y;
      s.z += o[j].z;
      s.w += o[j].w;
    }
  }
  if (ns) {  // the shared expert's output, weight 1
    s.x += osh.x;
    s.y += osh.y;
    s.z += osh.z;
    s.w += osh.w;
  }
  // the outputs of token t were formed from h 2^(2 a_t)
  const int e2 = -2 * ea;
  s = make_float4(ldexpf(s.x, e2), ldexpf(s.y, e2), ldexpf(s.z, e2), ldexpf(s.w, e2));
  if (resid) {
    float4 rv = rv0;
    rv.x += s.x;
    rv.y += s.y;
    rv.z += s.z;
    rv.w += s.w;
    *rp = rv;
  }
  if (y_out) *reinterpret_cast<float4*>(y_out + (size_t)t * d + r) = s;
}

// ----------------------------------------------------------------- launchers

template <int D>
static void prenorm_inst(const float* r, float eps, int T, uint16_t* xn, hipStream_t s) {
  hipLaunchKernelGGL((k_prenorm<D>), dim3(T), dim3(64), 0, s, r, eps, xn);
}

// Top-k (and, for T <= kTopkSortMax, the sort in the same kernel).
template <int EPL, int D>
static void topk_inst_d(const LayerArgs& a, const uint16_t* x, int T, int S, int32_t* idx_out, float* w_out,
                        hipStream_t s) {
  if (T <= kTopkSortMax) {
    const size_t lds = (size_t)5 * a.E * sizeof(int);
    const int g = (T + 3) / 4, CS = chunk_rows(a, T);
    if (a.k <= 8)
      hipLaunchKernelGGL((k_topk_sort<EPL, 8, D>), dim3(g), dim3(256), lds, s, a, x, T, S, idx_out, w_out, CS);
    else
      hipLaunchKernelGGL((k_topk_sort<EPL, 16, D>), dim3(g), dim3(256), lds, s, a, x, T, S, idx_out, w_out, CS);
    return;
  }
  if (a.k <= 8)
    hipLaunchKernelGGL((k_topk<EPL, 8, D>), dim3(T), dim3(64), 0, s, a, x, T, S, idx_out, w_out);
  else
    hipLaunchKernelGGL((k_topk<EPL, 16, D>), dim3(T), dim3(64), 0, s, a, x, T, S, idx_out, w_out);
}

template <int EPL>
static void topk_inst(const LayerArgs& a, const uint16_t* x, int T, int S, int32_t* idx_out, float* w_out,
                      hipStream_t s) {
  switch (a.d) {
    case 256: topk_inst_d<EPL, 256>(a, x, T, S, idx_out, w_out, s); break;
    case 512: topk_inst_d<EPL, 512>(a, x, T, S, idx_out, w_out, s); break;
    case 1024: topk_inst_d<EPL, 1024>(a, x, T, S, idx_out, w_out, s); break;
    case 2048: topk_inst_d<EPL, 2048>(a, x, T, S, idx_out, w_out, s); break;
    case 4096: topk_inst_d<EPL, 4096>(a, x, T, S, idx_out, w_out, s); break;
    default: topk_inst_d<EPL, 8192>(a, x, T, S, idx_out, w_out, s); break;
  }
}

hipError_t launch_router(const LayerArgs& a, const uint16_t* x, const float* r, float eps, int T,
                         int32_t* idx_out, float* w_out, uint16_t* x_trace, hipStream_t s) {
  if (!x) {  // the stack: pre-norm of the residual first
    uint16_t* xn = x_trace ? x_trace : a.xn;
    switch (a.d) {
      case 256: prenorm_inst<256>(r, eps, T, xn, s); break;
      case 512: prenorm_inst<512>(r, eps, T, xn, s); break;
      case 1024: prenorm_inst<1024>(r, eps, T, xn, s); break;
      case 2048: prenorm_inst<2048>(r, eps, T, xn, s); break;
      case 4096: prenorm_inst<4096>(r, eps, T, xn, s); break;
      case 8192: prenorm_inst<8192>(r, eps, T, xn, s); break;
      default: return hipErrorInvalidValue;
    }
    x = xn;
  }
  const int S = router_splits(T, a.E, a.d), nb = router_nb(T);
  const int grid = ((a.E + kRtE - 1) / kRtE) * ((T + 16 * nb - 1) / (16 * nb)) * S;
  switch (nb) {
    case 1: hipLaunchKernelGGL((k_router_mm<1>), dim3(grid), dim3(256), 0, s, a, x, T, S); break;
    case 2: hipLaunchKernelGGL((k_router_mm<2>), dim3(grid), dim3(256), 0, s, a, x, T, S); break;
    case 4: hipLaunchKernelGGL((k_router_mm<4>), dim3(grid), dim3(256), 0, s, a, x, T, S); break;
    default: hipLaunchKernelGGL((k_router_mm<8>), dim3(grid), dim3(256), 0, s, a, x, T, S); break;
  }
  const int epl = (a.E + 63) / 64;
  if (epl <= 1)
    topk_inst<1>(a, x, T, S, idx_out, w_out, s);
  else if (epl <= 2)
    topk_inst<2>(a, x, T, S, idx_out, w_out, s);
  else if (epl <= 4)
    topk_inst<4>(a, x, T, S, idx_out, w_out, s);
  else if (epl <= 8)
    topk_inst<8>(a, x, T, S, idx_out, w_out, s);
  else
    topk_inst<16>(a, x, T, S, idx_out, w_out, s);
  if (T <= kTopkSortMax) return hipGetLastError();  // sorted by the top-k kernel
  const size_t lds = sort_lds_bytes(a.E, T * a.k);
  if (lds > 64 * 1024) {
    static bool raised = false;
    if (!raised) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sort), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)sort_lds_bytes(1024, kMaxAssignments)) != hipSuccess)
        return hipErrorInvalidValue;
      raised = true;
    }
  }
  if (T * a.k >= kSortWideMin) {
    const size_t l4 = (size_t)4 * a.E * sizeof(int);
    hipLaunchKernelGGL(k_sort_count, dim3(kSortWideWaves / 4), dim3(256), l4, s, a, T);
    hipLaunchKernelGGL(k_sort_scan, dim3(1), dim3(1024), (size_t)a.E * sizeof(int), s, a, T, chunk_rows(a, T));
    hipLaunchKernelGGL(k_sort_place, dim3(kSortWideWaves / 4), dim3(256), l4, s, a, T);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_sort, dim3(1), dim3(1024), lds, s, a, T, chunk_rows(a, T));
  return hipGetLastError();
}

// Workgroup items: (chunk, row group); at most min(E, T*k) + T*k/CS chunks.
static int max_chunks(const LayerArgs& a, int T) {
  const int Tk = T * a.k, cs = chunk_rows(a, T);
  return (a.E < Tk ? a.E : Tk) + Tk / cs + a.ns * ((T + cs - 1) / cs);
}
// A multiple of 8 (one share per XCD), at most what stays resident.
static int grid_for(const LayerArgs& a, int T, int groups) {
  const int items = (max_chunks(a, T) * groups + 7) & ~7;
  return items < kMaxGroupedGrid ? items : kMaxGroupedGrid;
}

template <int NTT, int FMT>
static hipError_t gateup_inst(const LayerArgs& a, dim3 g, hipStream_t s) {
  const dim3 b(256);
  switch (a.d) {
    case 256: hipLaunchKernelGGL((k_gateup<256, NTT, FMT>), g, b, 0, s, a); break;
    case 512: hipLaunchKernelGGL((k_gateup<512, NTT, FMT>), g, b, 0, s, a); break;
    case 1024: hipLaunchKernelGGL((k_gateup<1024, NTT, FMT>), g, b, 0, s, a); break;
    case 2048: hipLaunchKernelGGL((k_gateup<2048, NTT, FMT>), g, b, 0, s, a); break;
    case 4096: hipLaunchKernelGGL((k_gateup<4096, NTT, FMT>), g, b, 0, s, a); break;
    case 8192: hipLaunchKernelGGL((k_gateup<8192, NTT, FMT>), g, b, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gateup(const LayerArgs& a, int T, hipStream_t s) {
  const dim3 g(grid_for(a, T, a.f / 64));
  const bool c64 = chunk_rows(a, T) == 64;
  if (a.fmt == 2) return c64 ? gateup_inst<4, 2>(a, g, s) : gateup_inst<2, 2>(a, g, s);
  if (a.fmt == 1) return c64 ? gateup_inst<4, 1>(a, g, s) : gateup_inst<2, 1>(a, g, s);
  return c64 ? gateup_inst<4, 0>(a, g, s) : gateup_inst<2, 0>(a, g, s);
}

template <int NTT, int FMT>
static hipError_t down_inst(const LayerArgs& a, dim3 g, hipStream_t s) {
  const dim3 b(256);
  switch (a.f) {
    case 128: hipLaunchKernelGGL((k_down<128, NTT, FMT>), g, b, 0, s, a); break;
    case 256: hipLaunchKernelGGL((k_down<256, NTT, FMT>), g, b, 0, s, a); break;
    case 512: hipLaunchKernelGGL((k_down<512, NTT, FMT>), g, b, 0, s, a); break;
    case 1024: hipLaunchKernelGGL((k_down<1024, NTT, FMT>), g, b, 0, s, a); break;
    case 2048: hipLaunchKernelGGL((k_down<2048, NTT, FMT>), g, b, 0, s, a); break;
    case 4096: hipLaunchKernelGGL((k_down<4096, NTT, FMT>), g, b, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The down kernel, then the combine (a kernel of its own: summing the slot
// outputs inside the down kernel, by the last item to finish each token's
// row group, made every item wait for its stores to reach the coherence
// point, an arrival count and the reads of the other slots' rows -- three
// round trips per item, measured slower than the extra kernel).
hipError_t launch_down_combine(const LayerArgs& a, int T, float* y_out, float* residual, hipStream_t s) {
  const dim3 g(grid_for(a, T, a.d / 128));
  const bool c64 = chunk_rows(a, T) == 64;
  hipError_t e;
  if (a.fmt == 2) e = c64 ? down_inst<4, 2>(a, g, s) : down_inst<2, 2>(a, g, s);
  else if (a.fmt == 1) e = c64 ? down_inst<4, 1>(a, g, s) : down_inst<2, 1>(a, g, s);
  else e = c64 ? down_inst<4, 0>(a, g, s) : down_inst<2, 0>(a, g, s);
  if (e != hipSuccess) return e;
  const int n4 = T * a.d / 4;
  const dim3 cg((n4 + 255) / 256), cb(256);
  if (a.k <= 1) hipLaunchKernelGGL(k_combine<1>, cg, cb, 0, s, a.obuf, a.xexp, T, a.d, a.k, a.ns, y_out, residual);
  else if (a.k <= 2) hipLaunchKernelGGL(k_combine<2>, cg, cb, 0, s, a.obuf, a.xexp, T, a.d, a.k, a.ns, y_out, residual);
  else if (a.k <= 4) hipLaunchKernelGGL(k_combine<4>, cg, cb, 0, s, a.obuf, a.xexp, T, a.d, a.k, a.ns, y_out, residual);
  else if (a.k <= 8) hipLaunchKernelGGL(k_combine<8>, cg, cb, 0, s, a.obuf, a.xexp, T, a.d, a.k, a.ns, y_out, residual);
  else hipLaunchKernelGGL(k_combine<16>, cg, cb, 0, s, a.obuf, a.xexp, T, a.d, a.k, a.ns, y_out, residual);
  return hipGetLastError();
}

// fmt: 0 int4, 1 MXFP4, 2 NVFP4 (tsc: its matrix scales, rows_per_mat rows each)
static hipError_t tile_matrix(const uint8_t* q, const uint16_t* sc, uint8_t* tq, uint16_t* ts, long long rows, int K,
                              int fmt, const float* tsc, long long rows_per_mat, hipStream_t s) {
  const long long np = rows * (K / 32), ns = rows * (K / 128);
  hipLaunchKernelGGL(k_tile_codes, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(q), reinterpret_cast<uint4*>(tq), rows, K);
  if (fmt == 2)
    hipLaunchKernelGGL(k_tile_scales_nv, dim3((unsigned)((2 * ns + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint8_t*>(sc), tsc, rows_per_mat, rows, K, reinterpret_cast<uint2*>(ts));
  else if (fmt == 1)
    hipLaunchKernelGGL((k_tile_scales<uint32_t>), dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t*>(sc), reinterpret_cast<uint32_t*>(ts), rows, K);
  else
    hipLaunchKernelGGL((k_tile_scales<uint2>), dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint2*>(sc), reinterpret_cast<uint2*>(ts), rows, K);
  return hipGetLastError();
}

// Bytes per 32 elements of the tile-major scale copy: 2 (int4 binary16), 1
// (MXFP4 E8M0), 4 (NVFP4: two fp16 per 32 elements).
static size_t copy_scale_bytes(int fmt) { return fmt == 1 ? 1 : fmt == 2 ? 4 : 2; }
static uint16_t* scales_at(const uint16_t* base, size_t n, int fmt) {
  return const_cast<uint16_t*>(
      reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(base) + n * copy_scale_bytes(fmt)));
}

hipError_t launch_tile_weights(const LayerArgs& a, hipStream_t s) {
  const long long E = a.E;
  hipError_t e;
  const size_t nt = (size_t)((E + 15) / 16) * (a.d / 32) * 64;
  hipLaunchKernelGGL(k_router_terms, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, s, a.router_w, a.E, a.d,
                     reinterpret_cast<uint4*>(const_cast<uint16_t*>(a.router_t)));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int fmt = a.fmt;
  const long long F = a.f, Dd = a.d;
  if ((e = tile_matrix(a.gate_q, a.gate_s, const_cast<uint8_t*>(a.gate_t), const_cast<uint16_t*>(a.gate_ts),
                       E * a.f, a.d, fmt, a.gate_tscale, F, s)) != hipSuccess)
    return e;
  if ((e = tile_matrix(a.up_q, a.up_s, const_cast<uint8_t*>(a.up_t), const_cast<uint16_t*>(a.up_ts), E * a.f,
                       a.d, fmt, a.up_tscale, F, s)) != hipSuccess)
    return e;
  if ((e = tile_matrix(a.down_q, a.down_s, const_cast<uint8_t*>(a.down_t), const_cast<uint16_t*>(a.down_ts),
                       E * a.d, a.f, fmt, a.down_tscale, Dd, s)) != hipSuccess)
    return e;
  if (!a.ns) return hipSuccess;
  // the shared expert as expert E of the copies (scale offsets in scales of 32 elements)
  const size_t gq = (size_t)E * a.f * a.d / 2, gs = (size_t)E * a.f * (a.d / 32);
  const size_t dq = (size_t)E * a.d * a.f / 2, ds = (size_t)E * a.d * (a.f / 32);
  if ((e = tile_matrix(a.sh_gate_q, a.sh_gate_s, const_cast<uint8_t*>(a.gate_t) + gq, scales_at(a.gate_ts, gs, fmt),
                       a.f, a.d, fmt, a.sh_gate_tscale, F, s)) != hipSuccess)
    return e;
  if ((e = tile_matrix(a.sh_up_q, a.sh_up_s, const_cast<uint8_t*>(a.up_t) + gq, scales_at(a.up_ts, gs, fmt), a.f,
                       a.d, fmt, a.sh_up_tscale, F, s)) != hipSuccess)
    return e;
  return tile_matrix(a.sh_down_q, a.sh_down_s, const_cast<uint8_t*>(a.down_t) + dq, scales_at(a.down_ts, ds, fmt),
                     a.d, a.f, fmt, a.sh_down_tscale, Dd, s);
}



}  // namespace moe
