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
// topk_fast selects with 32-bit keys holding the top bits of the
// order-preserving logit bits and, in the low bits, the inverted expert
// index, so keys are distinct and the largest names its owner.  The
// truncation can only mis-order logits that agree in their top bits; every
// consecutive pair of the k + 1 largest keys is checked and, if any agree,
// the selection is redone by topk_exact, which compares full values and
// breaks exact ties by ballot.
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

// Bitonic compare-exchange network sorting N registers in descending order
// (N a power of two), all indices compile-time.
template <int N>
__device__ __forceinline__ void sort_desc(uint32_t (&a)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;  // direction of this run
          const uint32_t hi = max(a[i], a[j]), lo = min(a[i], a[j]);
          a[i] = desc ? hi : lo;
          a[j] = desc ? lo : hi;
        }
      }
}

// a: descending; b: descending.  a receives the KP largest of both, descending.
template <int KP>
__device__ __forceinline__ void merge_top(uint32_t (&a)[KP], const uint32_t (&b)[KP]) {
#pragma unroll
  for (int i = 0; i < KP; ++i) a[i] = max(a[i], b[KP - 1 - i]);  // bitonic: falls, then rises
#pragma unroll
  for (int stride = KP >> 1; stride > 0; stride >>= 1)
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int j = i ^ stride;
      if (j > i) {
        const uint32_t hi = max(a[i], a[j]), lo = min(a[i], a[j]);
        a[i] = hi;
        a[j] = lo;
      }
    }
}

// The k choices (lane r < k gets choice r, every lane gets its own slot's
// expert through slot_e), the same as topk_exact unless it returns false
// (two of the k + 1 largest keys agree in their top bits; the caller must
// then use topk_exact).  k <= KP (a power of two <= 16).
// Selection by k rounds of wave maxima would chain k times about ten
// dependent DPP/permlane steps.  Here every lane sorts its EPL keys and the
// lanes merge their lists of the KP largest along the six pairing steps of
// a wave reduction (each step: the partner's list through DPP or a permlane
// swap, then a bitonic merge in registers), so every lane ends with the
// global KP largest, in order.
template <int EPL, int KP>
__device__ __forceinline__ bool topk_select_merge(const float v[EPL], int E, int k, int lane, int& sel_e) {
  const int ib = E <= 2 ? 1 : 32 - __clz(E - 1);
  const uint32_t imask = (1u << ib) - 1u;
  constexpr int N0 = EPL > KP ? EPL : KP;
  uint32_t a0[N0];
#pragma unroll
  for (int i = 0; i < N0; ++i)
    a0[i] = i < EPL && lane + 64 * i < E ? ((ordered_bits(v[i]) & ~imask) | (imask - (uint32_t)(lane + 64 * i))) : 0u;
  sort_desc<N0>(a0);
  uint32_t L[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) L[i] = a0[i];
  uint32_t P[KP];
#define TOPK_DPP_LEVEL(CTRL)                                \
  _Pragma("unroll") for (int i = 0; i < KP; ++i) P[i] = dpp_u<CTRL>(L[i]); \
  merge_top<KP>(L, P);
  TOPK_DPP_LEVEL(kDppXor1)
  TOPK_DPP_LEVEL(kDppXor2)
  TOPK_DPP_LEVEL(kDppHalfMirror)
  TOPK_DPP_LEVEL(kDppMirror)
#undef TOPK_DPP_LEVEL
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const u32x2_t p = swap16(L[i]);
    L[i] = p.x, P[i] = p.y;
  }
  merge_top<KP>(L, P);
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const u32x2_t p = swap32(L[i]);
    L[i] = p.x, P[i] = p.y;
  }
  merge_top<KP>(L, P);
  // every lane: L = the KP largest keys, descending
  uint32_t mine = 0, kth = 0, next = 0;
  bool close = false;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    mine = lane == i ? L[i] : mine;
    kth = i == k - 1 ? L[i] : kth;
    next = i == k ? L[i] : next;
    if (i >= 1) close = close || (i < k && ((L[i - 1] ^ L[i]) & ~imask) == 0u);
  }
  if (k == KP && k < E) {  // the best unchosen key is not in the lists
    uint32_t rest = 0;
#pragma unroll
    for (int i = 0; i < N0; ++i) rest = max(rest, a0[i] < kth ? a0[i] : 0u);
    next = wave_max_u32(rest);
  }
  close = close || (k < E && ((kth ^ next) & ~imask) == 0u);
  sel_e = lane < k ? (int)(imask - (mine & imask)) : 0;
  return !close;
}

// ---------------------------------------------------------------- block top-k
// The 256 threads of a workgroup hold one key each (expert e = thread,
// E <= 256).  Each wave sorts the 16 largest of its 64 keys across its
// lanes with a bitonic network (compare-exchange steps whose partner lane
// is i ^ M, reached by DPP or a permlane swap), the four lists meet in LDS,
// and two merge levels give every wave the 16 largest of all E, in lanes
// 0..15, descending.  About 30 steps of 3-4 VALU instructions each, instead
// of every wave merging lists of all 256 keys.

enum : int { kDppRev4 = 0x1B, kDppShr1 = 0x111 };

// The value of lane i ^ 16 (or i ^ 32): one of the pair a permlane swap
// returns is this lane's own value, the other the partner's.
__device__ __forceinline__ uint32_t partner16(uint32_t v) {
  const u32x2_t p = swap16(v);
  return p.x != v ? p.x : p.y;
}
__device__ __forceinline__ uint32_t partner32(uint32_t v) {
  const u32x2_t p = swap32(v);
  return p.x != v ? p.x : p.y;
}
// The value of lane i ^ M.
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (M == 1) return dpp_u<kDppXor1>(v);
  else if constexpr (M == 2) return dpp_u<kDppXor2>(v);
  else if constexpr (M == 3) return dpp_u<kDppRev4>(v);
  else if constexpr (M == 4) return dpp_u<kDppRev4>(dpp_u<kDppHalfMirror>(v));  // (i ^ 7) ^ 3
  else if constexpr (M == 7) return dpp_u<kDppHalfMirror>(v);
  else if constexpr (M == 8) return dpp_u<kDppHalfMirror>(dpp_u<kDppMirror>(v));  // (i ^ 15) ^ 7
  else if constexpr (M == 15) return dpp_u<kDppMirror>(v);
  else if constexpr (M == 31) return dpp_u<kDppMirror>(partner16(v));  // (i ^ 16) ^ 15
  else {
    static_assert(M == 47, "lane pattern");
    return dpp_u<kDppMirror>(partner32(v));  // (i ^ 32) ^ 15
  }
}
// Compare-exchange with lane i ^ M: the lane whose bit B is clear keeps the
// larger key, the other the smaller.
template <int M, int B>
__device__ __forceinline__ uint32_t cx(uint32_t v, int lane) {
  const uint32_t p = lane_xor<M>(v);
  return (lane >> B) & 1 ? min(v, p) : max(v, p);
}
// Lanes 0..15 of every 32: the 16 largest keys of the two sorted 16-lane
// groups 0..15 and 16..31 (M = 31, B = 4); or of lanes 0..15 and 32..47
// (M = 47, B = 5).  Bitonic: mirror step, then half-cleaners.
template <int M, int B>
__device__ __forceinline__ uint32_t merge16(uint32_t v, int lane) {
  v = cx<M, B>(v, lane);
  v = cx<8, 3>(v, lane);
  v = cx<4, 2>(v, lane);
  v = cx<2, 1>(v, lane);
  return cx<1, 0>(v, lane);
}
// key: this thread's key (0 for none).  s_top: 64 words of LDS.  Returns,
// in every wave, the 16 largest keys of the workgroup in lanes 0..15
// (descending; lanes 16..63 undefined).  Contains a barrier: every thread
// of the workgroup must call it.
__device__ __forceinline__ uint32_t block_top16(uint32_t key, int lane, int wid, uint32_t* s_top) {
  uint32_t v = key;
  // sorted runs of 2, 4, 8, 16 lanes
  v = cx<1, 0>(v, lane);
  v = cx<3, 1>(v, lane);
  v = cx<1, 0>(v, lane);
  v = cx<7, 2>(v, lane);
  v = cx<2, 1>(v, lane);
  v = cx<1, 0>(v, lane);
  v = cx<15, 3>(v, lane);
  v = cx<4, 2>(v, lane);
  v = cx<2, 1>(v, lane);
  v = cx<1, 0>(v, lane);
  // the wave's 16 largest in lanes 0..15
  v = merge16<31, 4>(v, lane);
  v = merge16<47, 5>(v, lane);
  if (lane < 16) s_top[16 * wid + lane] = v;
  __syncthreads();
  v = s_top[lane];  // the four waves' lists in lanes 0..15, 16..31, 32..47, 48..63
  v = merge16<31, 4>(v, lane);
  return merge16<47, 5>(v, lane);
}

// Faster selection with the same result as topk_exact (see above); k <= KP.
template <int EPL, int KP>
__device__ __forceinline__ void topk_fast(const float v[EPL], int E, int k, int norm, int lane, int& sel_e,
                                          float& sel_w) {
  if (!topk_select_merge<EPL, KP>(v, E, k, lane, sel_e)) {
    topk_exact<EPL>(v, E, k, norm, lane, sel_e, sel_w);
    return;
  }
  sel_w = topk_weight<EPL>(v, E, k, norm, lane, sel_e);
}

}  // namespace moe
