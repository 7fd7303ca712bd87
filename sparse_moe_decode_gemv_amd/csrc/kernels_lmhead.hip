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
// to arrive (a two-level count, below) reduces the G keys, writes token and
// max logit, and clears the top counter so the next call starts from zero.
#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace moe {

// Larger logit first, then the smaller row.
__device__ __forceinline__ unsigned long long make_key(float z, uint32_t row) {
  return ((unsigned long long)ordered_bits(z) << 32) | (unsigned long long)(0xFFFFFFFFu - row);
}

constexpr int kLmMaxGrid = 4096;

// Arrival.  Same-address atomics are serialized (about 14 ns each here), so
// G workgroups finishing together on one counter would end the kernel with G
// of them in a row.  Instead groups of kLmArr workgroups count on counters
// of their own, each on its own 128-byte line, and the last of each group
// counts on the top counter (line 0).  Every counter is zeroed by the last
// to arrive on it.  Called by one thread after the workgroup's partial
// results were stored and waited for; true in the last workgroup to arrive.
constexpr int kLmArr = 32;
constexpr int kLmLine = 32;  // counters are kLmLine unsigned apart
constexpr size_t kLmCtrBytes = ((1 + kLmMaxGrid / kLmArr) * 128 + 255) / 256 * 256;
__device__ __forceinline__ bool lm_arrive_last(unsigned* ctr) {
  const int G = gridDim.x, g = blockIdx.x / kLmArr, ng = (G + kLmArr - 1) / kLmArr;
  const unsigned gsize = (unsigned)min(kLmArr, G - g * kLmArr);
  unsigned* mine = ctr + (size_t)(1 + g) * kLmLine;
  if (arrive(mine) != gsize - 1) return false;
  __hip_atomic_store(mine, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return arrive(ctr) == (unsigned)ng - 1;
}

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

  // Tiles are dealt round-robin to the waves.  Every load is unconditional,
  // so the compiler's wait counts stay exact: in the last tile, pieces past
  // the matrix read its last piece (their rows are >= V and are dropped
  // below).  A tile's base is uniform (scalar registers) and lanes add
  // 32-bit offsets.  The 4 scales of piece c (pieces 4i .. 4i+3 of a row
  // hold the 4 groups 4i .. 4i+3) start at scale c & ~3.
  static_assert(CPR % 4 == 0, "pieces of a row come in fours");
  const size_t ntiles = (total + 64 * NL - 1) / (64 * NL), stride = (size_t)gridDim.x * 4;
  const size_t nfull = total / (64 * NL);
  auto load_tile = [&](size_t t, uint4 (&q)[NL], uint2 (&sc)[NL]) {
    const uint4* tq = wp + t * 64 * NL;
    const uint16_t* ts = ws + t * 64 * NL;
    if (t < nfull) {
#pragma unroll
      for (int n = 0; n < NL; ++n) {
        const uint32_t c = 64 * n + lane;
        q[n] = tq[c];
        sc[n] = *reinterpret_cast<const uint2*>(ts + (c & ~3u));
      }
    } else {
#pragma unroll
      for (int n = 0; n < NL; ++n) {
        const uint32_t c = (uint32_t)min((size_t)(64 * n + lane), total - 1 - t * 64 * NL);
        q[n] = tq[c];
        sc[n] = *reinterpret_cast<const uint2*>(ts + (c & ~3u));
      }
    }
  };
  // This wave's first tile is requested before x: the two round trips
  // overlap instead of following each other.  (The wave index goes through
  // readfirstlane so that the tile sequence is known to be uniform: scalar
  // loop control.)
  uint4 q[NL];
  uint2 sc[NL];
  const size_t t0 = (size_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(wid);
  if (t0 < ntiles) load_tile(t0, q, sc);

  // x row b enters as binary16 slices of x 2^xa[b], its largest magnitude
  // in [2^14, 2^15): the bf16 values are exact there down to 2^-24 of that
  // maximum, and the fp16 magic number takes one shift per dword where the
  // bf16 one takes three.  The argmax of a row is unchanged by the factor;
  // its maximum logit is scaled back at the end.  (Each wave's lanes cover
  // the whole row, so the wave maximum is the row's.)
  Slice8 xs[BP][XS][4];
  int xa[BP];
#pragma unroll
  for (int b = 0; b < BP; ++b) {
    uint4 xv[XS][4];
    uint32_t mb = 0;
#pragma unroll
    for (int s = 0; s < XS; ++s) {
      const int cc = CPR > 64 ? 64 * s + lane : lane % CPR;
      const int base = 128 * (cc >> 2) + 8 * (cc & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // rows past B read row B-1 and are zeroed once loaded (a load in
        // one arm of a branch makes the other arm's write of its registers
        // wait for it: the loads would run one at a time)
        const uint4 v = reinterpret_cast<const uint4*>(x + (size_t)min(b, B - 1) * D)[(base + 32 * j) >> 3];
        xv[s][j] = b < B ? v : make_uint4(0u, 0u, 0u, 0u);
        mb = max(mb, max(max(bf16_mag_max(xv[s][j].x), bf16_mag_max(xv[s][j].y)),
                         max(bf16_mag_max(xv[s][j].z), bf16_mag_max(xv[s][j].w))));
      }
    }
    xa[b] = act_exponent(wave_max_u32(mb)) + kXf16Shift;
#pragma unroll
    for (int s = 0; s < XS; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 q = xv[s][j];
        const float f[8] = {ldexpf(bf16_bits_to_f32(q.x & 0xFFFFu), xa[b]), ldexpf(__uint_as_float(q.x & 0xFFFF0000u), xa[b]),
                            ldexpf(bf16_bits_to_f32(q.y & 0xFFFFu), xa[b]), ldexpf(__uint_as_float(q.y & 0xFFFF0000u), xa[b]),
                            ldexpf(bf16_bits_to_f32(q.z & 0xFFFFu), xa[b]), ldexpf(__uint_as_float(q.z & 0xFFFF0000u), xa[b]),
                            ldexpf(bf16_bits_to_f32(q.w & 0xFFFFu), xa[b]), ldexpf(__uint_as_float(q.w & 0xFFFF0000u), xa[b])};
        xs[b][s][j] = make_slice_f16(f);
      }
  }

  float best[BP];
  uint32_t brow[BP];
#pragma unroll
  for (int b = 0; b < BP; ++b) best[b] = -INFINITY, brow[b] = 0xFFFFFFFFu;

  auto dot_tile = [&](size_t t, const uint4 (&q)[NL], const uint2 (&sc)[NL]) {
    const size_t c0 = t * 64 * NL;
    float acc[BP];
#pragma unroll
    for (int b = 0; b < BP; ++b) acc[b] = 0.f;
    if constexpr (CPR == 64 && BP == 1 && NL == 8) {
      // one row per piece column: the 8 row sums of the tile at once, lane
      // l holding row c0 / 64 + ((l >> 3) & 7)
      float z8[8];
#pragma unroll
      for (int n = 0; n < NL; ++n) z8[n] = dot_piece_f16(q[n], xs[0][0], sc[n]);
      const float z = wave_sum8_scatter(z8);
      const uint32_t row = (uint32_t)(c0 / 64) + ((lane >> 3) & 7);
      if (row < (uint32_t)V && z > best[0]) best[0] = z, brow[0] = row;
      return;
    }
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const int s = CPR > 64 ? n % XS : 0;
#pragma unroll
      for (int b = 0; b < BP; ++b) acc[b] += dot_piece_f16(q[n], xs[b][s], sc[n]);
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
  };
  for (size_t t = t0; t < ntiles; t += stride) {
    dot_tile(t, q, sc);
    if (t + stride < ntiles) load_tile(t + stride, q, sc);  // uniform branch
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
  if (threadIdx.x == 0) s_last = lm_arrive_last(counter);
  __syncthreads();
  if (!s_last) return;
  // last workgroup: reduce G keys per x row, every load issued before any
  // is waited for; 64-bit maxima within each wave (lane shuffles), then
  // over the 4 waves
#pragma unroll
  for (int b = 0; b < BP; ++b) {
    if (b >= B) break;
    constexpr int KL = kLmMaxGrid / 256;
    unsigned long long kv[KL];
#pragma unroll
    for (int m = 0; m < KL; ++m) {
      const int g = min(threadIdx.x + 256 * m, gridDim.x - 1);  // repeats past G: harmless for a maximum
      kv[m] = load_coherent(partial + (size_t)g * BP + b);
    }
    unsigned long long kmax = 0;
#pragma unroll
    for (int m = 0; m < KL; ++m) kmax = kv[m] > kmax ? kv[m] : kmax;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long t = __shfl_xor(kmax, o, 64);
      kmax = t > kmax ? t : kmax;
    }
    if (lane == 0) s_best[wid][0] = kmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long m = s_best[0][0];
#pragma unroll
      for (int w = 1; w < 4; ++w) m = s_best[w][0] > m ? s_best[w][0] : m;
      token[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFull));
      if (max_logit) max_logit[b] = ldexpf(unordered_bits((uint32_t)(m >> 32)), -xa[b]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) *counter = 0u;
}

// ---------------------------------------------------------------- MFMA path (2 <= B <= 16)
//
// Logits of 16 vocabulary rows x up to 16 x rows per group of 32 elements
// with one v_mfma_f32_16x16x32_f16 (A = x rows, zero past B; B operand = 16
// weight rows: lane l holds row l%16, chunk l/16 of the group).  A group of
// 32 is exactly one scale group, so the operand holds the codes q = u - 8
// (small integers, exact in fp16) and the scale is applied to the MFMA's
// fp32 result, accumulated in fp32: the weights enter exactly.  x enters as
// fp16 after multiplying each row by a power of two that brings its largest
// magnitude into [2^14, 2^15) (bf16 values are then exact in fp16 down to
// 2^-24 of the row maximum); the argmax of a row is unchanged by that
// factor and its maximum logit is scaled back at the end.
// One workgroup of 8 waves per compute unit: two groups of 4 waves, each
// group on its own sequence of tiles, the 4 waves of a group splitting K
// into quarters.  (Two 4-wave workgroups per compute unit would share it
// unevenly -- the older one's waves win arbitration and finish first, the
// other then runs alone at half the memory parallelism; the groups here
// step together, one barrier per tile pair.)  Each wave keeps its quarter
// of x as fragments in registers (elements in the order 0,4,1,5,2,6,3,7 of
// every 8, the order the magic-number extraction yields) and streams 16-row
// tiles of W with loads that are contiguous along each row (256 bytes of a
// row per quarter for d = 2048), two tiles ahead, the first two issued
// before x is read; a small wave-private LDS block, XOR-swizzled so that
// its stores and its fragment reads are free of bank conflicts, turns them
// into MFMA lane order.  The quarter sums meet in LDS; the first wave of
// each group keeps the running (value, row) maximum per x row.  Workgroup
// keys are stored row-major and the last workgroup to arrive reduces them
// with all its threads, every load issued before any is waited for.
typedef _Float16 lm_f16x8 __attribute__((ext_vector_type(8)));
typedef float lm_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lm_magic() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}
// 8 codes of one dword (elements e = 0..7, nibble e of the stored format) as
// fp16 q = u - 8 in the order e0,e4,e1,e5,e2,e6,e3,e7: the nibbles are
// placed in the mantissa of 1024 (even: 1024 + u; odd: 1024 + 16u) and the
// offset removed exactly
__device__ __forceinline__ lm_f16x8 lm_codes(uint32_t w, uint32_t magic) {
  const f16x2_t off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2_t sx = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2_t so = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w8 = w >> 8;
  const f16x2_t q0 = __builtin_bit_cast(f16x2_t, (w & 0x000F000Fu) | magic) + off;
  const f16x2_t q1 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, (w & 0x00F000F0u) | magic), sx, so);
  const f16x2_t q2 = __builtin_bit_cast(f16x2_t, (w8 & 0x000F000Fu) | magic) + off;
  const f16x2_t q3 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, (w8 & 0x00F000F0u) | magic), sx, so);
  const uint4 v = make_uint4(__builtin_bit_cast(uint32_t, q0), __builtin_bit_cast(uint32_t, q1),
                             __builtin_bit_cast(uint32_t, q2), __builtin_bit_cast(uint32_t, q3));
  return __builtin_bit_cast(lm_f16x8, v);
}
__device__ __forceinline__ uint32_t lm_dword(uint4 v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }

template <int D>
__global__ __launch_bounds__(512, 1) void k_lmhead_mfma(const uint8_t* __restrict__ wq,
                                                        const uint16_t* __restrict__ ws, int V,
                                                        const uint16_t* __restrict__ x, int B,
                                                        unsigned long long* __restrict__ partial,
                                                        unsigned* __restrict__ counter, int32_t* __restrict__ token,
                                                        float* __restrict__ max_logit) {
  constexpr int KQ = D / 4;          // K elements per wave
  constexpr int NBQ = KQ / 128;      // 128-element blocks per wave
  constexpr int PPR = KQ / 32;       // 16-byte pieces of a row in the quarter
  constexpr int RPI = 64 / PPR;      // rows per load instruction
  constexpr int NI = 16 / RPI;       // load instructions per 16-row tile
  constexpr int SH = 16 / PPR > 1 ? (16 / PPR == 2 ? 1 : 2) : 0;  // log2(16 / PPR)
  static_assert(NBQ >= 1 && PPR <= 64 && 64 % PPR == 0, "d = 512, 1024 or 2048");
  __shared__ uint4 s_w[8][16 * PPR];
  __shared__ uint2 s_s[8][16 * NBQ];
  __shared__ lm_f32x4 s_acc[2][8][64];
  __shared__ unsigned long long s_key[2][16];
  __shared__ uint4 s_x[16 * (D / 8 + 1)];
  __shared__ uint32_t s_xm2[16];
  __shared__ bool s_last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, q = lane >> 4;
  const int grp = wave >> 2, kq = wave & 3;  // tile group, K quarter
  const uint32_t magic = lm_magic();
  const int ntiles = (V + 15) >> 4;
  const int G2 = 2 * (int)gridDim.x;  // tiles of group grp: 2 * blockIdx + grp + n * G2

  // weight loads of one tile: instruction i, lane l -> row RPI*i + l/PPR of the tile, piece l%PPR
  struct TileRegs {
    uint4 w[NI];
    uint2 s;
  };
  auto load_tile = [&](int tt) {
    TileRegs r;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = min(16 * tt + RPI * i + lane / PPR, V - 1);
      r.w[i] = *reinterpret_cast<const uint4*>(wq + (size_t)row * (D / 2) + kq * (KQ / 2) + 16 * (lane % PPR));
    }
    const int srow = min(16 * tt + min(lane / NBQ, 15), V - 1);
    r.s = *reinterpret_cast<const uint2*>(ws + (size_t)srow * (D / 32) + kq * (KQ / 32) + 4 * (lane % NBQ));
    return r;
  };
  // x, staged once per workgroup: the 512 threads copy the B rows into LDS
  // (16 bytes each per pass; a row padded by 16 bytes so that the 16 rows
  // one fragment read touches fall in different banks) and take each row's
  // largest magnitude with LDS atomics
  constexpr int XC = D / 8;            // 16-byte chunks per row
  constexpr int XP = 16 * XC / 512;    // passes for 16 rows
  static_assert(XC % 64 == 0, "a wave's chunks of one pass in one row");
  if (tid < 16) s_xm2[tid] = 0u;
  uint4 xv[XP];
  // pass m reads chunk block (m + rot) % XP: the workgroups of one XCD
  // (every 8th) start on different blocks, so that 32 compute units do not
  // all miss on the same lines at once
  const int rot = (int)(blockIdx.x >> 3) % XP;
#pragma unroll
  for (int m = 0; m < XP; ++m) {
    const int mb = m + rot < XP ? m + rot : m + rot - XP;
    const int c = min(tid + 512 * mb, B * XC - 1);  // past the B rows: reread the last chunk, not stored
    xv[m] = *reinterpret_cast<const uint4*>(x + (size_t)c * 8);
  }
  __syncthreads();  // s_xm2 cleared
#pragma unroll
  for (int m = 0; m < XP; ++m) {
    // a wave's 64 chunks lie in one row (64 divides XC): one LDS atomic per wave
    const int mb = m + rot < XP ? m + rot : m + rot - XP;
    const int c = tid + 512 * mb, row = c / XC;
    uint32_t mm = 0;
    if (c < B * XC) {
      s_x[row * (XC + 1) + c % XC] = xv[m];
      const uint32_t cw[4] = {xv[m].x, xv[m].y, xv[m].z, xv[m].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) mm = max(mm, max(cw[e] & 0x7FFFu, (cw[e] >> 16) & 0x7FFFu));
    }
    mm = wave_max_u32(mm);  // largest |x| of the row as a bf16 magnitude pattern (ordered like the values)
    if (lane == 0 && row < B) atomicMax(&s_xm2[row], mm);
  }
  __syncthreads();
  const uint32_t xm = r16 < B ? s_xm2[r16] : 0u;
  // row r16 is multiplied by 2^-sh, sh = (exponent of its maximum) - 14
  const int sh = max((int)(xm >> 7) - 141, -126);
  const float fx = __uint_as_float((uint32_t)(127 - sh) << 23);
  // this wave's quarter of x as fp16 fragments: row r16 (zero past B), block b, group j, chunk q
  uint4 xf[NBQ][4];
#pragma unroll
  for (int b = 0; b < NBQ; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k0 = kq * KQ + 128 * b + 32 * j + 8 * q;
      uint4 v = s_x[min(r16, 15) * (XC + 1) + k0 / 8];
      if (r16 >= B) v = make_uint4(0, 0, 0, 0);
      const float e0 = bf16_bits_to_f32(v.x & 0xFFFFu) * fx, e1 = __uint_as_float(v.x & 0xFFFF0000u) * fx;
      const float e2 = bf16_bits_to_f32(v.y & 0xFFFFu) * fx, e3 = __uint_as_float(v.y & 0xFFFF0000u) * fx;
      const float e4 = bf16_bits_to_f32(v.z & 0xFFFFu) * fx, e5 = __uint_as_float(v.z & 0xFFFF0000u) * fx;
      const float e6 = bf16_bits_to_f32(v.w & 0xFFFFu) * fx, e7 = __uint_as_float(v.w & 0xFFFF0000u) * fx;
      xf[b][j] = make_uint4(pack_f16(e0, e4), pack_f16(e1, e5), pack_f16(e2, e6), pack_f16(e3, e7));
    }

  // only now the first two tiles: a compute unit's memory pipeline takes
  // requests in order, and the tiles' requests (20 MB across the chip)
  // would hold up the issue of everything behind them for microseconds.
  // Tile t's loads issue before tile t + G2's, the order the loop consumes
  // them in, so the waits before each step leave the later tile in flight.
  int t = 2 * (int)blockIdx.x + grp;
  TileRegs tr0 = load_tile(min(t, ntiles - 1));
  __builtin_amdgcn_sched_barrier(0);
  TileRegs tr1 = load_tile(min(t + G2, ntiles - 1));

  float best[4];
  uint32_t brow[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) best[v] = -INFINITY, brow[v] = 0xFFFFFFFFu;

  // one tile per group and step: its weights (TR = tr0 or tr1) through the
  // wave's LDS block into MFMAs, then the next-but-one tile's loads into the
  // same registers; PAR also selects the accumulator buffer, so one barrier
  // per step suffices.  The two steps are written out so that each register
  // set stays in place and the next tile's loads stay in flight.
#define LM_MFMA_STEP(TR, PAR)                                                                                   \
  {                                                                                                            \
    _Pragma("unroll") for (int i = 0; i < NI; ++i) {                                                           \
      const int r = RPI * i + lane / PPR, p = lane % PPR;                                                      \
      s_w[wave][r * PPR + (p ^ ((r >> SH) & (PPR - 1)))] = TR.w[i]; /* piece p of row r at slot p ^ (r >> SH) */ \
    }                                                                                                          \
    if (lane < 16 * NBQ) s_s[wave][lane] = TR.s;                                                               \
    /* other lanes of this wave read these slots: keep the compiler from moving   */                          \
    /* the reads above the stores (the wave's LDS operations run in order)        */                          \
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");                                                     \
    TR = load_tile(min(t + 2 * G2, ntiles - 1));                                                               \
    lm_f32x4 acc = {0.f, 0.f, 0.f, 0.f};                                                                       \
    _Pragma("unroll") for (int b = 0; b < NBQ; ++b) {                                                          \
      const int p = 4 * b + q;                                                                                 \
      const uint4 wc = s_w[wave][r16 * PPR + (p ^ ((r16 >> SH) & (PPR - 1)))];                                 \
      const uint2 sc = s_s[wave][r16 * NBQ + b];                                                               \
      const float sg[4] = {f16_lo(sc.x), f16_hi(sc.x), f16_lo(sc.y), f16_hi(sc.y)};                            \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                                          \
        const lm_f32x4 g = __builtin_amdgcn_mfma_f32_16x16x32_f16(                                             \
            __builtin_bit_cast(lm_f16x8, xf[b][j]), lm_codes(lm_dword(wc, j), magic),                          \
            lm_f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);                                                            \
        _Pragma("unroll") for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(sg[j], g[v], acc[v]);            \
      }                                                                                                        \
    }                                                                                                          \
    s_acc[PAR][wave][lane] = acc;                                                                              \
    __syncthreads();                                                                                           \
    if (kq == 0) {                                                                                             \
      /* lane: vocabulary row 16t + r16, x rows 4q + v */                                                      \
      const lm_f32x4 z = (s_acc[PAR][4 * grp][lane] + s_acc[PAR][4 * grp + 1][lane]) +                         \
                         (s_acc[PAR][4 * grp + 2][lane] + s_acc[PAR][4 * grp + 3][lane]);                      \
      const uint32_t row = 16u * t + r16;                                                                      \
      _Pragma("unroll") for (int v = 0; v < 4; ++v) if (row < (uint32_t)V && z[v] > best[v]) best[v] = z[v],   \
          brow[v] = row;                                                                                       \
    }                                                                                                          \
    t += G2;                                                                                                   \
  }
  // steps in pairs, as many as group 0 has tiles (group 1 has as many or one
  // fewer): a step past a group's last tile reads a clamped tile and updates
  // nothing; a single loop exit keeps the waits precise
  const int nsteps = (ntiles - 2 * (int)blockIdx.x + G2 - 1) / G2;
  for (int n = 0; n < nsteps; n += 2) {
    LM_MFMA_STEP(tr0, 0)
    LM_MFMA_STEP(tr1, 1)
  }
#undef LM_MFMA_STEP

  // per group and x row: maximum over the 16 lanes of its group (rows in increasing order per lane)
  if (kq == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      unsigned long long key = brow[v] == 0xFFFFFFFFu ? 0ull : make_key(best[v], brow[v]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const unsigned long long other = __shfl_xor(key, o, 64);
        key = other > key ? other : key;
      }
      if (r16 == 0) s_key[grp][4 * q + v] = key;
    }
  }
  __syncthreads();
  const int G = gridDim.x;
  if (tid < B) {
    const unsigned long long k0 = s_key[0][tid], k1 = s_key[1][tid];
    store_coherent(partial + (size_t)tid * G + blockIdx.x, k0 > k1 ? k0 : k1);  // row-major [B][G]
    wait_vm();
  }
  __syncthreads();
  if (tid == 0) s_last = lm_arrive_last(counter);
  __syncthreads();
  if (!s_last) return;
  // last workgroup: 32 threads per x row, each loading its keys at once
  {
    const int b = tid >> 5, l32 = tid & 31;
    unsigned long long kmax = 0;
    if (b < B) {
      constexpr int KL = 16;  // keys per thread, G <= 512
      unsigned long long kv[KL];
#pragma unroll
      for (int m = 0; m < KL; ++m) {
        const int g = min(l32 + 32 * m, G - 1);  // repeats past G: harmless for a maximum
        kv[m] = load_coherent(partial + (size_t)b * G + g);
      }
#pragma unroll
      for (int m = 0; m < KL; ++m) kmax = kv[m] > kmax ? kv[m] : kmax;
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const unsigned long long other = __shfl_xor(kmax, o, 64);
      kmax = other > kmax ? other : kmax;
    }
    if (b < B && l32 == 0) {
      token[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)(kmax & 0xFFFFFFFFull));
      if (max_logit) {
        max_logit[b] = ldexpf(unordered_bits((uint32_t)(kmax >> 32)), max((int)(s_xm2[b] >> 7) - 141, -126));
      }
    }
  }
  if (tid == 0) *counter = 0u;
}

size_t lmhead_workspace_bytes(int V, int d, int B) {
  (void)V;
  (void)d;
  const int launches = (B + 7) / 8;
  return (size_t)launches * (kLmCtrBytes + (size_t)kLmMaxGrid * 8 * sizeof(unsigned long long));
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
  unsigned long long* partial = reinterpret_cast<unsigned long long*>(wsp + kLmCtrBytes);
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

template <int D>
static hipError_t lm_mfma(const uint8_t* wq, const uint16_t* ws, int V, const uint16_t* x, int B, unsigned char* wsp,
                          int32_t* token, float* max_logit, hipStream_t s) {
  unsigned* counter = reinterpret_cast<unsigned*>(wsp);
  unsigned long long* partial = reinterpret_cast<unsigned long long*>(wsp + kLmCtrBytes);
  const int ntiles = (V + 15) / 16;
  int grid = lm_grid() / 4;  // one 8-wave workgroup per compute unit, at most kLmMaxGrid / 8
  if (grid > kLmMaxGrid / 8) grid = kLmMaxGrid / 8;
  if (grid > (ntiles + 1) / 2) grid = (ntiles + 1) / 2;
  hipLaunchKernelGGL((k_lmhead_mfma<D>), dim3(grid), dim3(512), 0, s, wq, ws, V, x, B, partial, counter, token,
                     max_logit);
  return hipGetLastError();
}

hipError_t launch_lmhead(const uint8_t* wq, const uint16_t* ws, int V, int d, const uint16_t* x, int B,
                         int32_t* token, float* max_logit, void* workspace, hipStream_t s) {
  unsigned char* wsp = static_cast<unsigned char*>(workspace);
  if (B >= 2 && B <= 16) {  // MFMA tiles (one 16-row x tile) for the shapes they are built for
    if (d == 512) return lm_mfma<512>(wq, ws, V, x, B, wsp, token, max_logit, s);
    if (d == 1024) return lm_mfma<1024>(wq, ws, V, x, B, wsp, token, max_logit, s);
    if (d == 2048) return lm_mfma<2048>(wq, ws, V, x, B, wsp, token, max_logit, s);
  }
  const size_t per = kLmCtrBytes + (size_t)kLmMaxGrid * 8 * sizeof(unsigned long long);
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

// ---------------------------------------------------------------- no-allocation variant
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the workspace is a file-scope device array of fixed size, one copy
// per GPU, held until the process ends.  Its address on each device is taken
// once, with that device current, through hipGetSymbolAddress; host code
// never passes the array's own name to a kernel (on the host it is only a
// stand-in for the symbol).  The arrival counters must be zero when a call
// starts: they are cleared by a fill kernel enqueued before the first call
// on each device, and every call leaves them at zero again.  Calls on one
// GPU share the array, so calls that overlap in time on one GPU race.
constexpr size_t kLmScratchBytes = 2 * (kLmCtrBytes + (size_t)kLmMaxGrid * 8 * sizeof(unsigned long long));
static __device__ __align__(256) unsigned char scratch[kLmScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device (set-up done)

__global__ void k_clear_u32(unsigned* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

size_t lmhead_scratch_bytes() { return kLmScratchBytes; }

hipError_t launch_lmhead_noalloc(const uint8_t* wq, const uint16_t* ws, int V, int d, const uint16_t* x, int B,
                                 int32_t* token, float* max_logit, hipStream_t s) {
  if (lmhead_workspace_bytes(V, d, B) > kLmScratchBytes) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev];
    if (!ptr) {  // set-up on this device: its copy's address, counters cleared
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      for (size_t c = 0; c < 2; ++c) {
        unsigned* ctr = reinterpret_cast<unsigned*>(static_cast<unsigned char*>(ptr) +
                                                    c * (kLmScratchBytes / 2));
        hipLaunchKernelGGL(k_clear_u32, dim3(16), dim3(256), 0, s, ctr, kLmCtrBytes / sizeof(unsigned));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      g_scratch_ptr[dev] = ptr;
    }
  }
  return launch_lmhead(wq, ws, V, d, x, B, token, max_logit, ptr, s);
}

}  // namespace moe
