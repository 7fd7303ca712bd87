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
//            carry this call's tag; every wave then runs the exact top-k
//            itself (lists of the largest keys merged across lanes in
//            registers, no serial rounds) and issues its gate/up loads;
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
// bounded: on timeout the kernel sets the error word and finishes anyway.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"
#include "topk.h"

namespace moe {

constexpr unsigned kSpinLimit = 1u << 21;
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
                            unsigned* error) {
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
    if (spin > kSpinLimit) {
      if (lane == 0) atomicOr(error, 1u);
      return;
    }
  }
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
template <int D, int F, int KP, int EPL, bool NORM, bool SH, int FMT>
__global__ __launch_bounds__(256) void k_layer(FusedArgs a) {
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
  static_assert(NL % LPRG == 0 && NI >= 1 && ROWS_G % 8 == 0, "shape");

  extern __shared__ unsigned s_sl[];  // k*F/8 slices x 5 words
  __shared__ int s_idx[16];
  __shared__ float s_w[16];
  __shared__ float s_part[4];
  __shared__ float s_hv[ROWS_G];
  __shared__ float s_lg[64 * EPL];
  __shared__ unsigned s_pub[ROWS_G / 8 * 5];

  __shared__ __align__(16) uint16_t s_x[D];
  __shared__ float s_ss[4];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wg = blockIdx.x * 4 + wid;
  const int E = a.E, k = a.k;
  const unsigned tag = a.epoch[blockIdx.x] + 1u;  // this workgroup's own call count
  const float bias = (a.router_b && wg < E) ? a.router_b[wg] : 0.f;

  // the activation in LDS: bf16 from the caller, or the normalized
  // residual.  Copied once at the start, so that no later phase issues a
  // global load behind the expert weight loads and waits for all of them.
  auto x2 = [&](int i) -> uint2 { return reinterpret_cast<const uint2*>(s_x)[i]; };  // elements 4i .. 4i+3
  auto x4 = [&](int i) -> uint4 { return reinterpret_cast<const uint4*>(s_x)[i]; };  // elements 8i .. 8i+7
  // router row wg (one per wave): its weight loads go out first and stay in
  // flight while the activation is staged
  const bool router_row = blockIdx.x * 4 < E && wg < E;
  float4 w[NI];
  if (router_row) {
    const float4* wr = reinterpret_cast<const float4*>(a.router_w + (size_t)wg * D);
#pragma unroll
    for (int i = 0; i < NI; ++i) w[i] = wr[64 * i + lane];
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
  auto load_mats = [&](const uint8_t* gq8, const uint16_t* gsb, const uint8_t* uq8, const uint16_t* usb) {
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
#pragma unroll
    for (int c = threadIdx.x; c < D / 8; c += 256) reinterpret_cast<uint4*>(s_x)[c] = reinterpret_cast<const uint4*>(a.x)[c];
    __syncthreads();
  } else {
    // x = bf16(r / sqrt(mean(r^2) + eps)), the same in every workgroup
    constexpr int NR = (D / 4 + 255) / 256;
    float4 rv[NR];
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int c = threadIdx.x + 256 * m;
      rv[m] = c < D / 4 ? reinterpret_cast<const float4*>(a.resid_in)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      ss = fmaf(rv[m].x, rv[m].x, ss);
      ss = fmaf(rv[m].y, rv[m].y, ss);
      ss = fmaf(rv[m].z, rv[m].z, ss);
      ss = fmaf(rv[m].w, rv[m].w, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) s_ss[wid] = ss;
    __syncthreads();
    const float den = sqrtf(((s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3])) / (float)D + a.eps);
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int c = threadIdx.x + 256 * m;
      if (c < D / 4) {
        const uint2 pk = make_uint2(pack_bf16(rv[m].x / den, rv[m].y / den), pack_bf16(rv[m].z / den, rv[m].w / den));
        reinterpret_cast<uint2*>(s_x)[c] = pk;
        if (a.x_trace && blockIdx.x == 0) reinterpret_cast<uint2*>(a.x_trace)[c] = pk;
      }
    }
    __syncthreads();
  }

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
  }

  // ---------------------------------------------------------------- select
  // wave 0 polls the logits and shares them through LDS; then every wave
  // runs the selection itself and issues its gate/up loads as soon as its
  // own slot is decided.  The softmax weights follow while the loads
  // are in flight (they are needed only at the end of gate/up).
  if (wid == 0) {
    float v0[EPL];
    poll_logits<EPL>(a.logits, E, tag, lane, v0, a.error);
#pragma unroll
    for (int i = 0; i < EPL; ++i) s_lg[lane + 64 * i] = v0[i];
  }
  __syncthreads();
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) v[i] = s_lg[lane + 64 * i];

  int se = 0;
  bool exact = false;
  if (topk_select_merge<EPL, KP>(v, E, k, lane, se)) {
    const int e_slot = __shfl(se, max(gslot, 0) & 63, 64);
    if (has_gate && !shared_slot) load_gate(e_slot);
  } else {  // picks that agree in their top bits: redo exactly
    float sw;
    topk_exact<EPL>(v, E, k, a.norm, lane, se, sw);
    if (wid == 0 && lane < k) s_w[lane] = sw;
    exact = true;
    const int e_slot = __shfl(se, max(gslot, 0) & 63, 64);
    if (has_gate && !shared_slot) load_gate(e_slot);
  }
  if (wid == 0) {
    if (lane < k) s_idx[lane] = se;
    if (!exact) {
      const float sw = topk_weight<EPL>(v, E, k, a.norm, lane, se);
      if (lane < k) s_w[lane] = sw;
    }
    __builtin_amdgcn_wave_barrier();
    if (blockIdx.x == 0 && lane < k) {
      if (a.idx_out) a.idx_out[lane] = se;
      if (a.w_out) a.w_out[lane] = s_w[lane];
    }
  }
  __syncthreads();

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
          if (lane == 0) s_hv[(wid * 64 * NL + 64 * n) / CPR] = wj * silu(g) * u;
        } else {
          const float g = seg_sum<(CPR < 64 ? CPR : 64)>(ag) * tg, u = seg_sum<(CPR < 64 ? CPR : 64)>(au) * tu;
          if (lane % CPR == 0) s_hv[(wid * 64 * NL + 64 * n + lane) / CPR] = wj * silu(g) * u;
        }
        ag = au = 0.f;
      }
    }
  }
  __syncthreads();
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
      if (writer) radd[n] = a.resid_in[row];
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

  // ---------------------------------------------------------------- collect h
  // all k*F/8 slices straight into LDS; a word is taken once it carries the
  // tag, and later polls re-read only the words still missing
  {
    constexpr int NR = (KP * F / 8 * 5 + 255) / 256;
    const int nw = nslots * (F / 8) * 5;  // slice words; word j = 5 * slice + field
    unsigned missing = 0;
#pragma unroll
    for (int m = 0; m < NR; ++m) missing |= (threadIdx.x + 256 * m < (unsigned)nw ? 1u : 0u) << m;
    for (unsigned spin = 0;; ++spin) {
      unsigned long long r[NR];
#pragma unroll
      for (int m = 0; m < NR; ++m)
        r[m] = (missing >> m) & 1u ? load_coherent(a.hrec + hrec_index(threadIdx.x + 256 * m, WPW, LPW)) : 0ull;
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        if (((missing >> m) & 1u) && (uint32_t)(r[m] >> 32) == tag) {
          s_sl[threadIdx.x + 256 * m] = (uint32_t)r[m];
          missing &= ~(1u << m);
        }
      }
      if (__syncthreads_or(missing != 0) == 0) break;
      if (spin > kSpinLimit) {
        if (threadIdx.x == 0) atomicOr(a.error, 2u);
        break;
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- down + combine
  auto put_y = [&](int row, float v, float r) {
    if constexpr (NORM) {
      a.resid_out[row] = r + v;
      if (a.y) a.y[row] = v;
    } else {
      a.y[row] = v;
    }
  };
  if (has_down) {
    Slice8 hs8[LPRD][4];
#pragma unroll
    for (int m = 0; m < LPRD; ++m) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = (act[m] ? dslot[m] : 0) * (F / 8) + 16 * (cc[m] >> 2) + 4 * j + (cc[m] & 3);
        const unsigned* sp = s_sl + 5 * c;
        hs8[m][j] = act[m] ? Slice8{sp[0], sp[1], sp[2], sp[3], __uint_as_float(sp[4])}
                           : Slice8{0u, 0u, 0u, 0u, 0.f};
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
          const float v = wave_sum(acc);
          if (lane == 0) put_y(r0 + n / LPRD, v, radd[n]);
        } else {
          const float v = seg_sum<(P < 64 ? P : 64)>(acc);
          if (lane % P == 0) put_y(r0 + n * RPLD + lane / P, v, radd[n]);
        }
        acc = 0.f;
      }
    }
  }
  if (threadIdx.x == 0) a.epoch[blockIdx.x] = tag;
}

// ---------------------------------------------------------------- launch chain (per format)

template <int D, int F, int KP, int EPL, int FMT>
static hipError_t layer_launch_fmt(const FusedArgs& a, int G, hipStream_t s) {
  const size_t lds = (size_t)(a.k + a.ns) * (F / 8) * 5 * sizeof(unsigned);
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

}  // namespace moe
