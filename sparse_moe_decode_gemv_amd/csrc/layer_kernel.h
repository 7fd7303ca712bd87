// layer_kernel.h -- the whole 1-token MoE layer step in one launch (gfx950):
// the kernel template and its launch chain, instantiated per weight format
// in kernels_layer.hip (int4), kernels_layer_mxfp4.hip and
// kernels_layer_nvfp4.hip (compiled side by side).
//
// Per token a small router picks a few of 256 routed experts and only those
// run ("Flint 40B: Best Mid Sized LLM", transcript 02:35).  The step is a
// chain of dependent phases -- router GEMV, top-k, expert gate/up + SwiGLU,
// down + combine -- and at one token each phase moves only a few MB, so the
// cost is latency, not bandwidth.  Measured on MI355X: a kernel boundary in
// a graph costs about 1.6 us, a counter-based grid barrier over 256
// workgroups about 3.7 us (same-address atomics serialize), and a coherent
// store is seen by a polling workgroup about 0.6 us later.  So this kernel
// keeps every workgroup resident (one per CU) and hands data between phases
// as self-validating words, with no atomics and no flags:
//
//   router   workgroup b computes router rows 4b..4b+3 (one per wave) and
//            writes the 4 logits as (tag << 32 | value) words into its own
//            128-byte line (one writer per line: words from different XCDs
//            sharing a line serialize at the memory side);
//   select   wave 0 of every workgroup polls the tagged logits until all
//            carry this call's tag; the workgroup's threads then key one
//            expert each and sort the 16 largest keys across lanes and
//            waves (topk.h, block_top16), so every wave knows the chosen
//            experts and issues its gate/up loads;
//   experts  the workgroup turns its 16 values h = w_j * silu(g) * u into
//            two ready-made fp16 dot slices and writes every slice word with
//            the tag, then prefetches its down pieces;
//   down     every workgroup polls all slice words straight into LDS until
//            they all carry the tag (the down pieces arrive meanwhile) and
//            finishes its output rows.
//
// In a pre-norm stack (NORM) the activation is not an input: every
// workgroup normalizes the fp32 residual itself (identical code and data,
// so identical bits) into LDS, and the output rows are added to the
// residual, read from one buffer and written to another so that no
// workgroup can see a row that another has already updated.
//
// The tag is this workgroup's call count + 1, kept per workgroup in the
// workspace; all workgroups take part in every call, so their counts agree
// and consecutive calls never accept each other's words.  Every wait is
// bounded (a.spin_limit polls): on timeout the kernel sets a bit of the
// error word, which the host reads through the library's error-flag call,
// and finishes anyway.  The waits assume that all G workgroups are resident
// at once (one per CU); if other work keeps some from starting, the waits
// time out instead of hanging.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"
#include "topk.h"

namespace moe {

// Phase timestamps, a diagnostic build only (-DMOE_PHASE_TRACE): thread 0
// of every workgroup stores the 100 MHz real-time counter at the marked
// points of the step (slots 0..10 of its 16); moe_decode_phase_trace copies
// the last call's values out.  Without the macro the marks compile to nothing.
#ifdef MOE_PHASE_TRACE
// one array per translation unit (one per weight format); the int4 one is
// read by phase_trace_copy
static __device__ unsigned long long g_phase_ts[kMaxFusedGrid * kPhaseSlots];
#define MOE_PHASE(i)                                                                                  \
  do {                                                                                                \
    if (threadIdx.x == 0) g_phase_ts[blockIdx.x * kPhaseSlots + (i)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define MOE_PHASE(i) \
  do {               \
  } while (0)
#endif

// Logits are published one 128-byte line per workgroup: words written by
// workgroups on different XCDs into one line serialize at the memory side
// (measured: all-to-all detection 2.2 us packed vs 1.3 us one line each).
constexpr int kLineWords64 = 16;

__device__ __forceinline__ void store_tagged(unsigned long long* p, float v, unsigned tag) {
  store_coherent(p, ((unsigned long long)tag << 32) | (unsigned long long)__float_as_uint(v));
}
// Every poll issues all of its coherent loads before looking at any result,
// so one poll costs one round trip to the coherence point, not one per load.

// Wave-wide: wait until the E tagged logits (4 per line) carry `tag`; v
// receives them (NaN mapped to -inf, entries past E to -inf).
template <int EPL>
__device__ void poll_logits(const unsigned long long* lg, int E, unsigned tag, int lane, float v[EPL],
                            unsigned* error, unsigned spin_limit) {
  for (unsigned spin = 0;; ++spin) {
    unsigned long long t[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = min(lane + 64 * i, E - 1);
      t[i] = load_coherent(lg + (size_t)(e >> 2) * kLineWords64 + (e & 3));
    }
    bool ok = true;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const bool valid = lane + 64 * i < E;
      const float f = __uint_as_float((uint32_t)t[i]);
      v[i] = valid && f == f ? f : -INFINITY;
      ok = ok & (!valid | ((uint32_t)(t[i] >> 32) == tag));
    }
    if (__builtin_amdgcn_ballot_w64(!ok) == 0) return;
    if (spin + 1 >= spin_limit) {
      if (lane == 0) atomicOr(error, 1u);
      return;
    }
  }
}

// Where a step takes x from and puts its output: the caller's x and y
// (kStepX); the residual r_l from memory, r_l + y written back (kStepNorm,
// one layer of a stack per launch); or, in a persistent stack, r_l from the
// previous layer's tagged words (from memory for the first layer) and
// r_l + y published as tagged words for the next layer (to memory after
// the last one) (kStepChain).
enum : int { kStepX = 0, kStepNorm = 1, kStepChain = 2 };

// The per-call inputs and outputs of one layer step.
struct StepIO {
  const uint16_t* x;              // kStepX: bf16 [D]
  const float* resid_in;          // kStepNorm, first kStepChain layer: r_l [D]
  const unsigned long long* rin;  // later kStepChain layers: the previous layer's tagged r words
  unsigned rin_tag;               //   and their tag
  float* resid_out;               // kStepNorm, last kStepChain layer: r_l + y [D]
  unsigned long long* rout;       // other kStepChain layers: this layer's tagged r words
  float eps;
  uint16_t* x_trace;              // x_l [D] (stack), or NULL
  float* y;                       // y [D] (kStepX), or a trace of it, or NULL
  int32_t* idx_out;               // [k] or NULL
  float* w_out;                   // [k] or NULL
  unsigned spin_limit, tag_skew;
  const float* next_router;       // kStepChain: the next layer's router matrix, or NULL
  int next_E;
};

// Residual word of row `row`: rows_per_wg consecutive rows per producing
// workgroup, in lines of their own.
__device__ __forceinline__ size_t rrec_index(int row, int rows_per_wg) {
  const int lpw = (rows_per_wg + 15) / 16;
  return (size_t)(row / rows_per_wg) * lpw * 16 + (row % rows_per_wg);
}

// Slice word j (= 5 * slice + field, slices in h order) sits in the lines of
// the workgroup that produced it: wpw words per workgroup, lpw lines each.
__device__ __forceinline__ size_t hrec_index(int j, int wpw, int lpw) {
  return (size_t)(j / wpw) * lpw * 16 + (j % wpw);
}

// D hidden, F expert width, KP expert slots (top_k, plus one with a shared
// expert, SH) rounded up to a power of two, EPL
// experts per lane in the top-k wave; FMT: expert weights int4 with binary16
// scales (0), MXFP4 (1: E2M1 codes, an E8M0 scale byte per 32) or NVFP4 (2:
// E2M1 codes, an E4M3 scale byte per 16, an fp32 scale per matrix).
template <int D, int F, int KP, int EPL, int MODE, bool SH, int FMT, class A>
__device__ __forceinline__ unsigned layer_step(const A& a, const StepIO& io, float4 (&w)[D / 256], bool w_ready) {
  constexpr bool NORM = MODE != kStepX;  // x is the normalized residual
  constexpr bool FP4 = FMT != 0, NV = FMT == 2;
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
  constexpr int NI = D / 256;        // router float4 per lane (one row per wave)
  constexpr int ROWS_G = 64 * NL / CPR * 4;  // gate/up rows per workgroup (C2: 16)
  constexpr int RPG = 4 * ROWS_W;             // output rows per workgroup (C2: 8)
  static_assert(NL % LPRG == 0 && NI >= 1 && ROWS_G % 8 == 0, "shape");

  // the KP*F/8 slices of h as the down phase reads them: p0..p3 of the
  // slice read at (m, j) by lane l at position (4m + j) * 64 + l (or
  // j * P + l % P when a row has fewer than 64 pieces), and its corr word
  // at the same position of a second array, so that each read is one
  // 16-byte (or 4-byte) load per lane at consecutive addresses
  extern __shared__ unsigned s_dyn[];
  uint4* s_slp = reinterpret_cast<uint4*>(s_dyn);
  float* s_slc = reinterpret_cast<float*>(s_dyn + 4 * KP * F / 8);
  __shared__ int s_idx[16];
  __shared__ float s_w[16];
  __shared__ float s_part[4];
  __shared__ float s_hv[ROWS_G];
  __shared__ float s_lg[64 * EPL];
  __shared__ uint32_t s_top[64];
  __shared__ float s_z[4];
  __shared__ unsigned s_pub[ROWS_G / 8 * 5];

  __shared__ __align__(16) uint16_t s_x[D];
  __shared__ __align__(16) float s_r[NORM ? D : 4];  // the residual r_l (stack)
  __shared__ float s_ss[4];
  __shared__ uint32_t s_xm[4];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wg = blockIdx.x * 4 + wid;
  const int E = a.E, k = a.k;
  const unsigned tag = a.epoch[blockIdx.x] + 1u;  // this workgroup's own call count
  const float bias = (a.router_b && wg < E) ? a.router_b[wg] : 0.f;
  MOE_PHASE(0);

  // the activation in LDS: bf16 from the caller, or the normalized
  // residual.  Copied once at the start, so that no later phase issues a
  // global load behind the expert weight loads and waits for all of them.
  auto x2 = [&](int i) -> uint2 { return reinterpret_cast<const uint2*>(s_x)[i]; };  // elements 4i .. 4i+3
  auto x4 = [&](int i) -> uint4 { return reinterpret_cast<const uint4*>(s_x)[i]; };  // elements 8i .. 8i+7
  // The activation (or the residual it is normalized from) is requested
  // first and the router row wg (one per wave) right behind it: a wave's
  // loads complete in order, so the activation's few bytes arrive one round
  // trip after the start and are staged (or normalized) while the router
  // rows are still streaming in, instead of after them.
  constexpr int XPT = (D / 8 + 255) / 256;  // 8-element x chunks per thread
  constexpr int NR = (D / 4 + 255) / 256;   // residual float4 per thread
  uint4 xq[XPT];
  float4 rv[NR];
  if constexpr (!NORM) {
#pragma unroll
    for (int m = 0; m < XPT; ++m) {
      const int c = threadIdx.x + 256 * m;
      xq[m] = c < D / 8 ? reinterpret_cast<const uint4*>(io.x)[c] : make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
#pragma unroll
    for (int m = 0; m < NR; ++m) rv[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (MODE == kStepNorm || !io.rin) {  // r from memory
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        const int c = threadIdx.x + 256 * m;
        if (c < D / 4) rv[m] = reinterpret_cast<const float4*>(io.resid_in)[c];
      }
    }
  }
  // Every wave issues the NI router loads (a wave without a router row
  // reads one 16-byte word NI times): with the same number of loads in
  // flight on every path the compiler waits for the activation alone
  // (vmcnt(NI)); with a branch around the router loads it has to wait for
  // all of them.
  const bool router_row = blockIdx.x * 4 < E && wg < E;
  if (!w_ready) {
    const float4* wr = reinterpret_cast<const float4*>(a.router_w) + (router_row ? (size_t)wg * (D / 4) + lane : 0);
#pragma unroll
    for (int i = 0; i < NI; ++i) w[i] = wr[router_row ? 64 * i : 0];
  }
  // gate/up slots: the k chosen experts, then the shared one (ns = 1), wpe
  // waves each
  const int wpe = (F * CPR) / (64 * NL);  // waves per expert slot
  const int nslots = k + (SH ? 1 : 0);
  const bool has_gate = wg < nslots * wpe;
  const int gslot = has_gate ? wg / wpe : -1;
  const bool shared_slot = SH && gslot >= k;
  const int c0 = has_gate ? (wg - gslot * wpe) * 64 * NL : 0;
  uint4 qg[NL], qu[NL];
  uint2 sg[NL], su[NL];
  // The 4 scales of piece c of row `row` (CP pieces per row): 4 binary16
  // (int4), 4 E8M0 bytes (MXFP4, in .x), or the 8 NVFP4 E4M3 bytes of the
  // piece's group (nv_scales picks the piece's 4 where they are used: no
  // arithmetic on a loaded value before the dot, which would make the wave
  // wait for it -- and for every load issued before it -- right away).
  auto load_scales = [&](const uint16_t* base, size_t row, int CP, int c) -> uint2 {
    if constexpr (NV) {
      return *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(base) + row * 2 * CP + 8 * (c >> 2));
    } else if constexpr (FP4) {
      return make_uint2(
          *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(base) + row * CP + (c & ~3)), 0u);
    } else {
      return *reinterpret_cast<const uint2*>(base + row * CP + (c & ~3));
    }
  };
  // scale array of expert e: e_off scales of 2 bytes (int4), 1 (MXFP4) or 2
  // per 32 elements (NVFP4)
  auto scales_of = [&](const uint16_t* base, size_t e_off) -> const uint16_t* {
    if constexpr (NV) return reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(base) + 2 * e_off);
    else if constexpr (FP4) return reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(base) + e_off);
    else return base + e_off;
  };
  float tg = 1.f, tu = 1.f;  // NVFP4 matrix scales of this wave's slot
  // NVFP4: piece c's E4M3 bytes of its group's 8 at bytes 0, 2, 4, 6
  auto nv_scales = [](uint2 v, int c) -> uint2 {
    const uint64_t s = (((uint64_t)v.y << 32) | v.x) >> (8 * ((c & 3) >> 1));
    return make_uint2((uint32_t)s, (uint32_t)(s >> 32));
  };
  // The slot's loads.  With x from the caller, as 32-bit lane offsets from
  // the matrices' uniform bases (the address arithmetic sits between the
  // top-k and the loads): piece c at byte 16 c, its scales at (c & ~3)
  // times the scale bytes per 32 elements -- 2 (int4, NVFP4: the group's 8
  // E4M3 bytes start there) or 1 (MXFP4) -- since pieces 4i .. 4i+3 of a row
  // hold its groups 4i .. 4i+3 (CPR is a multiple of 4).  Measured in one
  // process: 11.53 -> 11.11 us per step there, but 12.25 -> 12.49 us per
  // layer in the pre-normed stack kernel and 12.42 -> 12.99 in the
  // persistent one, whose schedules the compiler builds differently; those
  // keep the index form.
  static_assert(CPR % 4 == 0, "pieces of a row come in fours");
  auto load_mats = [&](const uint8_t* gq8, const uint16_t* gsb, const uint8_t* uq8, const uint16_t* usb) {
    if constexpr (MODE != kStepX) {
      const uint4* gp = reinterpret_cast<const uint4*>(gq8);
      const uint4* up = reinterpret_cast<const uint4*>(uq8);
#pragma unroll
      for (int n = 0; n < NL; ++n) {
        const int c = c0 + 64 * n + lane;
        qg[n] = gp[c];
        qu[n] = up[c];
        sg[n] = load_scales(gsb, (size_t)(c / CPR), CPR, c % CPR);
        su[n] = load_scales(usb, (size_t)(c / CPR), CPR, c % CPR);
      }
      return;
    }
    constexpr uint32_t SB = (FP4 && !NV) ? 1u : 2u;
    const uint8_t* gs8 = reinterpret_cast<const uint8_t*>(gsb);
    const uint8_t* us8 = reinterpret_cast<const uint8_t*>(usb);
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const uint32_t c = (uint32_t)(c0 + 64 * n + lane), so = SB * (c & ~3u);
      qg[n] = *reinterpret_cast<const uint4*>(gq8 + 16u * c);
      qu[n] = *reinterpret_cast<const uint4*>(uq8 + 16u * c);
      if constexpr (FP4 && !NV) {
        sg[n] = make_uint2(*reinterpret_cast<const uint32_t*>(gs8 + so), 0u);
        su[n] = make_uint2(*reinterpret_cast<const uint32_t*>(us8 + so), 0u);
      } else {
        sg[n] = *reinterpret_cast<const uint2*>(gs8 + so);
        su[n] = *reinterpret_cast<const uint2*>(us8 + so);
      }
    }
  };
  auto load_gate = [&](int e_raw) {
    const int e = min(max(e_raw, 0), E - 1);
    const size_t mat = (size_t)F * CPR;
    load_mats(a.gate_q + (size_t)e * mat * 16, scales_of(a.gate_s, (size_t)e * mat), a.up_q + (size_t)e * mat * 16,
              scales_of(a.up_s, (size_t)e * mat));
    if constexpr (NV) {
      tg = a.gate_tscale[e];
      tu = a.up_tscale[e];
    }
  };
  // the shared expert needs no routing: its slot's loads go out now, behind
  // the router rows, and land while the logits are exchanged
  if constexpr (SH)
    if (shared_slot) {
      load_mats(a.sh_gate_q, a.sh_gate_s, a.sh_up_q, a.sh_up_s);
      if constexpr (NV) {
        tg = a.sh_gate_tscale[0];
        tu = a.sh_up_tscale[0];
      }
    }
  if constexpr (!NORM) {
    uint32_t mb = 0;  // the largest |x| (bf16 bits)
#pragma unroll
    for (int m = 0; m < XPT; ++m) {
      const int c = threadIdx.x + 256 * m;
      if (c < D / 8) {
        const uint4 q = xq[m];
        reinterpret_cast<uint4*>(s_x)[c] = q;
        mb = max(mb, max(max(bf16_mag_max(q.x), bf16_mag_max(q.y)), max(bf16_mag_max(q.z), bf16_mag_max(q.w))));
      }
    }
    mb = wave_max_u32(mb);
    if (lane == 0) s_xm[wid] = mb;
    __syncthreads();
  } else {
    // x = bf16(r / sqrt(mean(r^2) + eps)), the same in every workgroup; r
    // from memory was requested at the start
    if (MODE == kStepChain && io.rin) {  // r from the previous layer's tagged words, each thread the 4 * NR it normalizes
      unsigned missing = 0;
#pragma unroll
      for (int m = 0; m < NR; ++m) missing |= (threadIdx.x + 256 * m < D / 4 ? 0xFu : 0u) << (4 * m);
      const unsigned want = io.rin_tag + io.tag_skew;
      for (unsigned spin = 0;; ++spin) {
        unsigned long long t[4 * NR];
#pragma unroll
        for (int i = 0; i < 4 * NR; ++i) {
          const int e = 4 * (threadIdx.x + 256 * (i / 4)) + i % 4;
          t[i] = (missing >> i) & 1u ? load_coherent(io.rin + rrec_index(min(e, D - 1), RPG)) : 0ull;
        }
#pragma unroll
        for (int i = 0; i < 4 * NR; ++i) {
          if (((missing >> i) & 1u) && (uint32_t)(t[i] >> 32) == want) {
            const float f = __uint_as_float((uint32_t)t[i]);
            float4& r4 = rv[i / 4];
            if (i % 4 == 0) r4.x = f;
            else if (i % 4 == 1) r4.y = f;
            else if (i % 4 == 2) r4.z = f;
            else r4.w = f;
            missing &= ~(1u << i);
          }
        }
        if (__syncthreads_or(missing != 0) == 0) break;
        if (spin + 1 >= io.spin_limit) {
          if (threadIdx.x == 0) atomicOr(a.error, 4u);
          break;
        }
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int c = threadIdx.x + 256 * m;
      if (c < D / 4) reinterpret_cast<float4*>(s_r)[c] = rv[m];
      ss = fmaf(rv[m].x, rv[m].x, ss);
      ss = fmaf(rv[m].y, rv[m].y, ss);
      ss = fmaf(rv[m].z, rv[m].z, ss);
      ss = fmaf(rv[m].w, rv[m].w, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) s_ss[wid] = ss;
    __syncthreads();
    // one reciprocal of the root, then products (within an ulp of the
    // quotients before the bf16 rounding)
    const float inv = 1.0f / sqrtf(((s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3])) / (float)D + io.eps);
    uint32_t mb = 0;
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int c = threadIdx.x + 256 * m;
      if (c < D / 4) {
        const uint2 pk = make_uint2(pack_bf16(rv[m].x * inv, rv[m].y * inv), pack_bf16(rv[m].z * inv, rv[m].w * inv));
        reinterpret_cast<uint2*>(s_x)[c] = pk;
        mb = max(mb, max(bf16_mag_max(pk.x), bf16_mag_max(pk.y)));
        if (io.x_trace && blockIdx.x == 0) reinterpret_cast<uint2*>(io.x_trace)[c] = pk;
      }
    }
    mb = wave_max_u32(mb);
    if (lane == 0) s_xm[wid] = mb;
    __syncthreads();
  }
  MOE_PHASE(1);  // x (or the normalized residual) in LDS
  // h goes to the down phase as h 2^(2 ea) in binary16, ea from the largest
  // |x| (the same in every workgroup): exact scalings, any magnitude of x
  const int ea = act_exponent(max(max(s_xm[0], s_xm[1]), max(s_xm[2], s_xm[3])));

  // ---------------------------------------------------------------- router
  // rows 4*b .. 4*b+3 in workgroup b, one per wave; the 4 logits go out as
  // (tag, value) words in the workgroup's own 128-byte line.
  if (blockIdx.x * 4 < E) {
    if (router_row) {
      uint2 q[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) q[i] = x2(64 * i + lane);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        acc = fmaf(w[i].x, bf16_bits_to_f32(q[i].x & 0xFFFFu), acc);
        acc = fmaf(w[i].y, __uint_as_float(q[i].x & 0xFFFF0000u), acc);
        acc = fmaf(w[i].z, bf16_bits_to_f32(q[i].y & 0xFFFFu), acc);
        acc = fmaf(w[i].w, __uint_as_float(q[i].y & 0xFFFF0000u), acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) s_part[wid] = acc + bias;
    }
    __syncthreads();
    if (threadIdx.x < 4 && blockIdx.x * 4 + (int)threadIdx.x < E)
      store_tagged(a.logits + (size_t)blockIdx.x * kLineWords64 + threadIdx.x, s_part[threadIdx.x], tag);
    MOE_PHASE(2);  // router workgroups: logits stored
  }

  // ---------------------------------------------------------------- select
  // wave 0 polls the logits and shares them through LDS; then every wave
  // runs the selection itself and issues its gate/up loads as soon as its
  // own slot is decided.  The softmax weights follow while the loads
  // are in flight (they are needed only at the end of gate/up).
  if (wid == 0) {
    float v0[EPL];
    poll_logits<EPL>(a.logits, E, tag + io.tag_skew, lane, v0, a.error, io.spin_limit);
#pragma unroll
    for (int i = 0; i < EPL; ++i) s_lg[lane + 64 * i] = v0[i];
  }
  __syncthreads();
  MOE_PHASE(3);  // every wave has the logits
  int se = 0;     // lanes 0..k-1: the chosen experts, larger logit first
  float sw = 0.f; // their weights
  const int gsl = __builtin_amdgcn_readfirstlane(max(gslot, 0));  // this wave's slot (uniform)
  bool fast = false;
  if (k < 16) {
    // every thread keys its expert; the 16 largest keys reach every wave
    const int ib = E <= 2 ? 1 : 32 - __clz(E - 1);
    const uint32_t imask = (1u << ib) - 1u;
    const int t = threadIdx.x;
    const float lt = t < E ? s_lg[t] : -INFINITY;
    const uint32_t key = t < E ? ((ordered_bits(lt) & ~imask) | (imask - (uint32_t)t)) : 0u;
    const uint32_t top = block_top16(key, lane, wid, s_top);
    MOE_PHASE(4);
    // two of the k + 1 largest keys that agree above the index bits may be
    // out of order: then the exact selection below decides
    const uint32_t prev = dpp_u<kDppShr1>(top);
    fast = __builtin_amdgcn_ballot_w64(lane >= 1 && lane <= k && ((prev ^ top) & ~imask) == 0u) == 0ull;
    if (fast) {
      se = lane < k ? (int)(imask - (top & imask)) : 0;
      if (has_gate && !shared_slot) load_gate(__builtin_amdgcn_readlane(se, gsl));
      MOE_PHASE(5);  // this wave's gate/up loads issued
      // weights while the loads fly: lane 0 holds the largest logit
      const float l = s_lg[se];
      const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 0));
      const float pe = lane < k ? expf(l - m) : 0.f;
      float den;
      if (a.norm) {
        den = seg_sum<16>(pe);  // lanes 0..15 (k <= 15)
      } else {  // the softmax's sum over all E experts
        const float z = wave_sum(t < E ? expf(lt - m) : 0.f);
        if (lane == 0) s_z[wid] = z;
        __syncthreads();
        den = (s_z[0] + s_z[1]) + (s_z[2] + s_z[3]);
      }
      sw = pe / den;
    }
  }
  if (!fast) {
    float v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = s_lg[lane + 64 * i];
    if (k < 16 || !topk_select_merge<EPL, KP>(v, E, k, lane, se)) {  // picks that agree in their top bits: redo exactly
      topk_exact<EPL>(v, E, k, a.norm, lane, se, sw);
      if (has_gate && !shared_slot) load_gate(__builtin_amdgcn_readlane(se, gsl));
    } else {
      if (has_gate && !shared_slot) load_gate(__builtin_amdgcn_readlane(se, gsl));
      sw = topk_weight<EPL>(v, E, k, a.norm, lane, se);
    }
  }
  if (wid == 0) {
    if (lane < k) {
      s_idx[lane] = se;
      s_w[lane] = sw;
    }
    if (blockIdx.x == 0 && lane < k) {
      if (io.idx_out) io.idx_out[lane] = se;
      if (io.w_out) io.w_out[lane] = sw;
    }
  }
  __syncthreads();
  MOE_PHASE(6);

  // ---------------------------------------------------------------- gate/up + SwiGLU
  if (has_gate) {
    const float wj = shared_slot ? 1.f : s_w[gslot];
    Slice8 xs[XS][4];
#pragma unroll
    for (int s = 0; s < XS; ++s) {
      const int c = CPR > 64 ? 64 * s + lane : lane % CPR;
      const int base = 128 * (c >> 2) + 8 * (c & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (FP4) xs[s][j] = make_slice_raw(x4((base + 32 * j) >> 3));
        else xs[s][j] = make_slice_bf16(x4((base + 32 * j) >> 3));
      }
    }
    float ag = 0.f, au = 0.f;
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const int s = CPR > 64 ? n % XS : 0;
      if constexpr (NV) {
        const int c = (c0 + 64 * n + lane) % CPR;
        ag += dot_piece_nv(qg[n], xs[s], nv_scales(sg[n], c));
        au += dot_piece_nv(qu[n], xs[s], nv_scales(su[n], c));
      } else if constexpr (FP4) {
        ag += dot_piece_fp4(qg[n], xs[s], sg[n].x);
        au += dot_piece_fp4(qu[n], xs[s], su[n].x);
      } else {
        ag += dot_piece(qg[n], xs[s], sg[n]);
        au += dot_piece(qu[n], xs[s], su[n]);
      }
      if (n % LPRG == LPRG - 1) {
        // row within this workgroup's ROWS_G consecutive rows of slot gslot
        if constexpr (CPR >= 64) {
          const float g = wave_sum(ag) * tg, u = wave_sum(au) * tu;
          if (lane == 0) s_hv[(wid * 64 * NL + 64 * n) / CPR] = wj * silu_scaled(g, ea) * ldexpf(u, ea);
        } else {
          const float g = seg_sum<(CPR < 64 ? CPR : 64)>(ag) * tg, u = seg_sum<(CPR < 64 ? CPR : 64)>(au) * tu;
          if (lane % CPR == 0) s_hv[(wid * 64 * NL + 64 * n + lane) / CPR] = wj * silu_scaled(g, ea) * ldexpf(u, ea);
        }
        ag = au = 0.f;
      }
    }
  }
  __syncthreads();
  MOE_PHASE(7);  // gate/up and SwiGLU done
  // publish this workgroup's rows as ready-made fp16 dot slices, one per 8
  // consecutive h values, every 64-bit word carrying the tag; the
  // workgroup's words fill its own 128-byte line(s), written by consecutive
  // lanes of one store instruction
  constexpr int SPW = ROWS_G / 8;          // slices per workgroup
  constexpr int WPW = SPW * 5;             // words per workgroup
  constexpr int LPW = (WPW + 15) / 16;     // 128-byte lines per workgroup
  const bool producer = blockIdx.x * 4 < nslots * wpe;
  if (producer && threadIdx.x < SPW) {
    float hv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] = s_hv[8 * threadIdx.x + e];
    const Slice8 sl = FP4 ? make_slice_f16_raw(hv) : make_slice_f16(hv);
    s_pub[5 * threadIdx.x + 0] = sl.p0, s_pub[5 * threadIdx.x + 1] = sl.p1, s_pub[5 * threadIdx.x + 2] = sl.p2;
    s_pub[5 * threadIdx.x + 3] = sl.p3, s_pub[5 * threadIdx.x + 4] = __float_as_uint(sl.corr);
  }
  __syncthreads();
  if (producer && wid == 0) {
    unsigned long long* line = a.hrec + (size_t)blockIdx.x * LPW * 16;  // producer index == workgroup index
    for (int w0 = 0; w0 < WPW; w0 += 64)
      if (w0 + lane < WPW) store_coherent(line + w0 + lane, ((unsigned long long)tag << 32) | s_pub[w0 + lane]);
  }
  MOE_PHASE(8);  // h published

  // ---------------------------------------------------------------- down prefetch
  // issued now so that the 4.7 MB of down pieces stream in while the h
  // hand-off is in flight, instead of competing with the gate/up loads
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
    act[m] = has_down && dslot[m] < nslots;
  }
  float td[LPRD];  // NVFP4: the matrix scale of each piece's expert (1 otherwise)
#pragma unroll
  for (int m = 0; m < LPRD; ++m) {
    td[m] = 1.f;
    if constexpr (NV) {
      if (act[m]) td[m] = (SH && dslot[m] >= k) ? a.sh_down_tscale[0] : a.down_tscale[min(max(s_idx[dslot[m]], 0), E - 1)];
    }
  }
  float radd[NLD];  // residual rows this lane will update (stack)
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    const int row = r0 + (P >= 64 ? n / LPRD : n * RPLD + lane / P);
    const bool writer = has_down && (P >= 64 ? lane == 0 : lane % P == 0) && n % LPRD == LPRD - 1;
    radd[n] = 0.f;
    if constexpr (NORM)
      if (writer) radd[n] = s_r[row];
  }
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    const int m = n % LPRD;
    const int row = r0 + (P >= 64 ? n / LPRD : n * RPLD + lane / P);
    if (act[m]) {
      const bool shd = SH && dslot[m] >= k;  // the shared expert's slot
      const size_t eb = shd ? (size_t)row : (size_t)min(max(s_idx[dslot[m]], 0), E - 1) * D + row;
      qd[n] = *reinterpret_cast<const uint4*>((shd ? a.sh_down_q : a.down_q) + piece_offset(eb, CPRF, cc[m]));
      sd[n] = load_scales(shd ? a.sh_down_s : a.down_s, eb, CPRF, cc[m]);
    } else {
      qd[n] = make_uint4(0, 0, 0, 0);
      sd[n] = make_uint2(0, 0);
    }
  }

  // the next layer's router rows (a persistent stack): loaded while this
  // layer's h is exchanged, ready when its activation is.  (With one launch
  // per layer, loading them here only to warm the caches for the next
  // launch measured slower: 12.23 -> 12.47 us per layer, the extra loads
  // completing ahead of the h polls.)
  if constexpr (MODE == kStepChain)
    if (io.next_router && blockIdx.x * 4 < io.next_E && wg < io.next_E) {
      const float4* wr = reinterpret_cast<const float4*>(io.next_router + (size_t)wg * D);
#pragma unroll
      for (int i = 0; i < NI; ++i) w[i] = wr[64 * i + lane];
    }

  // ---------------------------------------------------------------- collect h
  // all k*F/8 slices straight into LDS; a word is taken once it carries the
  // tag, and later polls re-read only the words still missing
  {
    constexpr int NR = (KP * F / 8 * 5 + 255) / 256;
    const int nw = nslots * (F / 8) * 5;  // slice words; word j = 5 * slice + field
    unsigned missing = 0;
    unsigned dst[NR];  // where word j goes in LDS (s_dyn words)
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int jw = threadIdx.x + 256 * m;
      missing |= (jw < nw ? 1u : 0u) << m;
      const int sl = jw / 5, fld = jw - 5 * sl;
      const int slot = sl / (F / 8), sidx = sl % (F / 8);
      const int flat = slot * CPRF + 4 * (sidx / 16) + (sidx & 3), jg = (sidx >> 2) & 3;  // piece, group of the slice
      const int pos = P >= 64 ? ((flat / 64) * 4 + jg) * 64 + flat % 64 : jg * P + flat;
      dst[m] = fld < 4 ? 4 * pos + fld : 4 * KP * F / 8 + pos;
    }
    for (unsigned spin = 0;; ++spin) {
      unsigned long long r[NR];
#pragma unroll
      for (int m = 0; m < NR; ++m)
        r[m] = (missing >> m) & 1u ? load_coherent(a.hrec + hrec_index(threadIdx.x + 256 * m, WPW, LPW)) : 0ull;
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        if (((missing >> m) & 1u) && (uint32_t)(r[m] >> 32) == tag + io.tag_skew) {
          s_dyn[dst[m]] = (uint32_t)r[m];
          missing &= ~(1u << m);
        }
      }
      if (__syncthreads_or(missing != 0) == 0) break;
      if (spin + 1 >= io.spin_limit) {
        if (threadIdx.x == 0) atomicOr(a.error, 2u);
        break;
      }
    }
    __syncthreads();
    MOE_PHASE(9);  // all h in LDS
  }

  // ---------------------------------------------------------------- down + combine
  auto put_y = [&](int row, float v, float r) {
    if constexpr (MODE == kStepChain) {
      if (io.y) io.y[row] = v;
      if (io.rout) store_tagged(io.rout + rrec_index(row, RPG), r + v, tag);  // to every workgroup
      else io.resid_out[row] = r + v;
    } else if constexpr (NORM) {
      io.resid_out[row] = r + v;
      if (io.y) io.y[row] = v;
    } else {
      io.y[row] = v;
    }
  };
  if (has_down) {
    Slice8 hs8[LPRD][4];
#pragma unroll
    for (int m = 0; m < LPRD; ++m) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pos = P >= 64 ? (4 * m + j) * 64 + lane : j * P + lane % P;
        const uint4 pv = s_slp[pos];
        const float cv = s_slc[pos];
        hs8[m][j] = act[m] ? Slice8{pv.x, pv.y, pv.z, pv.w, cv} : Slice8{0u, 0u, 0u, 0u, 0.f};
      }
    }
    float acc = 0.f;
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int m = n % LPRD;
      if constexpr (NV) acc = fmaf(dot_piece_nv_f16(qd[n], hs8[m], nv_scales(sd[n], cc[m])), td[m], acc);
      else if constexpr (FP4) acc += dot_piece_fp4_f16(qd[n], hs8[m], sd[n].x);
      else acc += dot_piece_f16(qd[n], hs8[m], sd[n]);
      if (n % LPRD == LPRD - 1) {
        if constexpr (P >= 64) {
          const float v = ldexpf(wave_sum(acc), -2 * ea);
          if (lane == 0) put_y(r0 + n / LPRD, v, radd[n]);
        } else {
          const float v = ldexpf(seg_sum<(P < 64 ? P : 64)>(acc), -2 * ea);
          if (lane % P == 0) put_y(r0 + n * RPLD + lane / P, v, radd[n]);
        }
        acc = 0.f;
      }
    }
  }
  MOE_PHASE(10);
  if (threadIdx.x == 0) a.epoch[blockIdx.x] = tag;
  return tag;
}


// One layer: x from the caller (NORM false) or the normalized residual of a
// stack (NORM true), arguments in the kernel's own argument block.
template <int D, int F, int KP, int EPL, bool NORM, bool SH, int FMT>
__global__ __launch_bounds__(256) void k_layer(FusedArgs a) {
  StepIO io{};
  io.x = a.x, io.resid_in = a.resid_in, io.resid_out = a.resid_out, io.eps = a.eps;
  io.x_trace = a.x_trace, io.y = a.y, io.idx_out = a.idx_out, io.w_out = a.w_out;
  io.spin_limit = a.spin_limit, io.tag_skew = a.tag_skew;
  float4 w[D / 256];
  layer_step<D, F, KP, EPL, NORM ? kStepNorm : kStepX, SH, FMT>(a, io, w, false);
}

// A persistent stack: every workgroup runs the L layers in turn (the
// single-launch analogue of the pages' decode mega-kernel, "Flint 40B: Best
// Mid Sized LLM", transcript 06:43: no launch between layers, and the next
// layer's router rows load while the current layer's h is exchanged).  The
// residual crosses from layer to layer as tagged words in the producing
// layer's workspace; each layer's arguments are read from the copy that
// init wrote into its workspace.
typedef const __attribute__((address_space(4))) FusedArgs ConstFusedArgs;

template <int D, int F, int KP, int EPL, bool SH, int FMT>
__global__ __launch_bounds__(256) void k_stack(StackArgs s) {
  float4 w[D / 256];
  unsigned tag = 0;
  const unsigned long long* rin = nullptr;
  for (int l = 0; l < s.L; ++l) {
    ConstFusedArgs& a = *(ConstFusedArgs*)s.layer[l];
    const bool last = l + 1 == s.L;
    StepIO io{};
    io.resid_in = s.resid_in, io.rin = rin, io.rin_tag = tag;
    io.resid_out = s.resid_out, io.rout = last ? nullptr : a.rrec;
    io.eps = s.eps;
    io.x_trace = s.x_trace ? s.x_trace + (size_t)l * D : nullptr;
    io.y = s.y_trace ? s.y_trace + (size_t)l * D : nullptr;
    io.idx_out = s.idx_trace ? s.idx_trace + (size_t)l * a.k : nullptr;
    io.spin_limit = s.spin_limit, io.tag_skew = s.tag_skew;
    if (!last) {
      ConstFusedArgs& n = *(ConstFusedArgs*)s.layer[l + 1];
      io.next_router = n.router_w, io.next_E = n.E;
    }
    tag = layer_step<D, F, KP, EPL, kStepChain, SH, FMT>(a, io, w, l > 0);
    rin = a.rrec;
  }
}

// ---------------------------------------------------------------- launch chain (per format)

template <int D, int F, int KP, int EPL, int FMT>
static hipError_t layer_launch_fmt(const FusedArgs& a, int G, hipStream_t s) {
  const size_t lds = (size_t)KP * (F / 8) * 5 * sizeof(unsigned);
  if (a.ns) {
    if (a.resid_in)
      hipLaunchKernelGGL((k_layer<D, F, KP, EPL, true, true, FMT>), dim3(G), dim3(256), lds, s, a);
    else
      hipLaunchKernelGGL((k_layer<D, F, KP, EPL, false, true, FMT>), dim3(G), dim3(256), lds, s, a);
  } else {
    if (a.resid_in)
      hipLaunchKernelGGL((k_layer<D, F, KP, EPL, true, false, FMT>), dim3(G), dim3(256), lds, s, a);
    else
      hipLaunchKernelGGL((k_layer<D, F, KP, EPL, false, false, FMT>), dim3(G), dim3(256), lds, s, a);
  }
  return hipGetLastError();
}

template <int FMT, int D, int F, int KP>
static hipError_t layer_epl(const FusedArgs& a, int G, hipStream_t s) {
  if (a.E <= 64) return layer_launch_fmt<D, F, KP, 1, FMT>(a, G, s);
  if (a.E <= 128) return layer_launch_fmt<D, F, KP, 2, FMT>(a, G, s);
  return layer_launch_fmt<D, F, KP, 4, FMT>(a, G, s);
}

template <int FMT, int D, int F>
static hipError_t layer_kp(const FusedArgs& a, int G, hipStream_t s) {
  const int k = a.k + a.ns;  // expert slots
  if (k <= 1) return layer_epl<FMT, D, F, 1>(a, G, s);
  if (k <= 2) return layer_epl<FMT, D, F, 2>(a, G, s);
  if (k <= 4) return layer_epl<FMT, D, F, 4>(a, G, s);
  if (k <= 8) return layer_epl<FMT, D, F, 8>(a, G, s);
  return layer_epl<FMT, D, F, 16>(a, G, s);
}

// The kernel of weight format FMT for the shapes it is built for.
template <int FMT>
static hipError_t launch_layer_format(const FusedArgs& a, int d, int f, int G, hipStream_t s) {
  if (d == 256 && f == 128) return layer_kp<FMT, 256, 128>(a, G, s);
  if (d == 2048 && f == 512) return layer_kp<FMT, 2048, 512>(a, G, s);
  return hipErrorInvalidValue;
}

// The persistent stack kernel for the shape `sh` (all of the launch's
// layers have it).
template <int D, int F, int KP, int EPL, int FMT>
static hipError_t stack_launch_fmt(const StackArgs& a, const StackShape& sh, int G, hipStream_t s) {
  const size_t lds = (size_t)KP * (F / 8) * 5 * sizeof(unsigned);
  if (sh.ns)
    hipLaunchKernelGGL((k_stack<D, F, KP, EPL, true, FMT>), dim3(G), dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL((k_stack<D, F, KP, EPL, false, FMT>), dim3(G), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int FMT, int D, int F, int KP>
static hipError_t stack_epl(const StackArgs& a, const StackShape& sh, int G, hipStream_t s) {
  if (sh.E <= 64) return stack_launch_fmt<D, F, KP, 1, FMT>(a, sh, G, s);
  if (sh.E <= 128) return stack_launch_fmt<D, F, KP, 2, FMT>(a, sh, G, s);
  return stack_launch_fmt<D, F, KP, 4, FMT>(a, sh, G, s);
}

template <int FMT, int D, int F>
static hipError_t stack_kp(const StackArgs& a, const StackShape& sh, int G, hipStream_t s) {
  const int k = sh.k + sh.ns;
  if (k <= 1) return stack_epl<FMT, D, F, 1>(a, sh, G, s);
  if (k <= 2) return stack_epl<FMT, D, F, 2>(a, sh, G, s);
  if (k <= 4) return stack_epl<FMT, D, F, 4>(a, sh, G, s);
  if (k <= 8) return stack_epl<FMT, D, F, 8>(a, sh, G, s);
  return stack_epl<FMT, D, F, 16>(a, sh, G, s);
}

template <int FMT>
static hipError_t launch_stack_format(const StackArgs& a, const StackShape& sh, int G, hipStream_t s) {
  if (sh.d == 256 && sh.f == 128) return stack_kp<FMT, 256, 128>(a, sh, G, s);
  if (sh.d == 2048 && sh.f == 512) return stack_kp<FMT, 2048, 512>(a, sh, G, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
