// topk.h -- exact softmax + top-k over E router logits in one wave (gfx950).
//
// The pages: per token a small router selects a few of the 256 routed
// experts ("Flint 40B: Best Mid Sized LLM", transcript 02:35).  Selection
// here is exact: the k largest logits (equivalently the k largest softmax
// probabilities), larger first, the lower expert index on equal logits.
//
// Each lane holds EPL logits (expert lane + 64*i).  Weights: p_j =
// exp(l_j - max l) over the chosen set, divided by their sum (renormalized)
// or by the sum over all experts.
//
// topk_fast: every round is one wave maximum (DPP + permlane, VALU only) of
// 32-bit keys holding the top bits of the order-preserving logit bits and,
// in the low bits, the inverted expert index, so the maximum names its
// owner.  The truncation can only mis-order logits that agree in their top
// bits; one extra round checks every consecutive pair of picks (the k-th
// against the best unpicked included) and, if any agree, the selection is
// redone by topk_exact, which compares full values and breaks exact ties by
// ballot.
#pragma once

#include "device_common.h"

namespace moe {

// v: this lane's logits (NaN already mapped to -inf); entries with
// lane + 64*i >= E are ignored.  Lane r < k ends with choice r in
// (sel_e, sel_w).
template <int EPL>
__device__ __forceinline__ void topk_exact(const float v[EPL], int E, int k, int norm, int lane, int& sel_e,
                                           float& sel_w) {
  uint32_t key[EPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const bool valid = lane + 64 * i < E;
    key[i] = valid ? ordered_bits(v[i]) : 0u;  // 0 sorts below every real key, -inf included
    m = valid ? fmaxf(m, v[i]) : m;
  }
  m = wave_max(m);
  float z = 0.f;
  if (!norm) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) z += lane + 64 * i < E ? expf(v[i] - m) : 0.f;
    z = wave_sum(z);
  }
  int my_e = 0;
  uint32_t my_key = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t loc = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) loc = max(loc, key[i]);
    const uint32_t M = wave_max_u32(loc);
    int e_sel = -1;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint64_t b = __builtin_amdgcn_ballot_w64(key[i] == M);
      if (e_sel < 0 && b) e_sel = (int)__builtin_ctzll(b) + 64 * i;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = lane + 64 * i == e_sel ? 0u : key[i];
    if (lane == r) {
      my_e = e_sel;
      my_key = M;
    }
  }
  const float p = lane < k ? expf(unordered_bits(my_key) - m) : 0.f;
  const float den = norm ? wave_sum(p) : z;
  sel_e = my_e;
  sel_w = p / den;
}

// Weights of the chosen experts: lane r < k holds choice e, its logit is
// fetched from the lane that holds it.
template <int EPL>
__device__ __forceinline__ float topk_weight(const float v[EPL], int E, int k, int norm, int lane, int my_e) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) m = lane + 64 * i < E ? fmaxf(m, v[i]) : m;
  m = wave_max(m);
  float z = 0.f;
  if (!norm) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) z += lane + 64 * i < E ? expf(v[i] - m) : 0.f;
    z = wave_sum(z);
  }
  float l_sel = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const float c = __shfl(v[i], my_e & 63, 64);
    l_sel = (my_e >> 6) == i ? c : l_sel;
  }
  const float p = lane < k ? expf(l_sel - m) : 0.f;
  const float den = norm ? wave_sum(p) : z;
  return p / den;
}

// The k choices only (lane r < k gets choice r), same result as topk_exact.
// Returns false when two picks agree in their top bits: the caller must then
// use topk_exact.
template <int EPL>
__device__ __forceinline__ bool topk_select_fast(const float v[EPL], int E, int k, int lane, int& sel_e) {
  const int ib = E <= 2 ? 1 : 32 - __clz(E - 1);
  const uint32_t imask = (1u << ib) - 1u;
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    key[i] = lane + 64 * i < E ? ((ordered_bits(v[i]) & ~imask) | (imask - (uint32_t)(lane + 64 * i))) : 0u;
  int my_e = 0;
  uint32_t prev = 0;
  bool close = false;
  for (int r = 0; r <= k && r < E; ++r) {
    uint32_t loc = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) loc = max(loc, key[i]);
    const uint32_t M = wave_max_u32(loc);
    close = close || (r > 0 && ((M ^ prev) & ~imask) == 0u);
    prev = M;
    if (r == k) break;
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = key[i] == M ? 0u : key[i];
    if (lane == r) my_e = (int)(imask - (M & imask));
  }
  sel_e = my_e;
  return !close;
}

// Faster selection with the same result as topk_exact (see above).
template <int EPL>
__device__ __forceinline__ void topk_fast(const float v[EPL], int E, int k, int norm, int lane, int& sel_e,
                                          float& sel_w) {
  if (!topk_select_fast<EPL>(v, E, k, lane, sel_e)) {
    topk_exact<EPL>(v, E, k, norm, lane, sel_e, sel_w);
    return;
  }
  sel_w = topk_weight<EPL>(v, E, k, norm, lane, sel_e);
}

}  // namespace moe
