// launch.h -- host-side launchers of the decode kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_decode.h"

namespace moe {

// Device pointers of one MoE layer plus the per-call workspace carve-up.
struct LayerArgs {
  int d, f, E, k, norm_topk;
  int ns;  // shared experts, 0 or 1: expert index E of the tile-major copies, assignments T*k + t
  int fmt;  // 0 int4; 1 MXFP4 (the *_s pointers and scale copies hold E8M0 bytes); 2 NVFP4 (E4M3 bytes per 16)
  int chunk_cap;  // entries of the chunk table (its size for max_tokens tokens)
  const float* gate_tscale;  // NVFP4: fp32 scale of each expert matrix [E] (shared: [1])
  const float* up_tscale;
  const float* down_tscale;
  const float* sh_gate_tscale;
  const float* sh_up_tscale;
  const float* sh_down_tscale;
  const float* router_w;
  const float* router_b;
  const uint8_t* gate_q;
  const uint16_t* gate_s;
  const uint8_t* up_q;
  const uint16_t* up_s;
  const uint8_t* down_q;
  const uint16_t* down_s;
  const uint8_t* sh_gate_q;  // the shared expert (ns = 1), formats as one expert of the above
  const uint16_t* sh_gate_s;
  const uint8_t* sh_up_q;
  const uint16_t* sh_up_s;
  const uint8_t* sh_down_q;
  const uint16_t* sh_down_s;
  // tile-major copies of the expert matrices, [E + ns] (batched path; max_tokens > 1):
  // codes in MFMA lane order (1 KB per 16 rows x 128 k); scales per (16 rows x 128 k)
  // as 16 rows of 4 binary16 (int4), 4 E8M0 bytes (MXFP4), or two sets of 4
  // binary16 block scales with the matrix scale folded in (NVFP4)
  const uint8_t* gate_t;
  const uint16_t* gate_ts;
  const uint8_t* up_t;
  const uint16_t* up_ts;
  const uint8_t* down_t;
  const uint16_t* down_ts;
  // three bf16 terms of the router matrix (h + m + l = W_r), MFMA tiles
  // [ceil(E/16)][d/32][term][64 lanes][8] (batched path)
  const uint16_t* router_t;
  // workspace of the batched path
  float* logits;          // [S][T][E16] router partial sums of S slices of K, E16 = E rounded up to 16
  uint16_t* xn;           // [T][d] pre-normed activations of a stack layer (bf16), unless x_trace holds them
  int32_t* sel_idx;       // [T][k] chosen experts of assignment t*k + j
  float* sel_w;           // [T][k] their weights
  uint16_t* xp;           // [T][d] activations x 2^a_t in MFMA operand order (fp16)
  int32_t* xexp;          // [T] a_t: the power of two that puts token t's largest |x| in [1, 2)
  int32_t* off;           // [E+1] first position of each expert in asg
  int32_t* act;           // [E] experts with assignments, ascending
  int32_t* chunk_off;     // [E+1] 32-token chunks of the active experts before each
  int4* chunks;           // [min(E, T*k) + T*k/32 + ns*ceil(T/32)] (expert, first position, count <= CS),
                          // CS = 32, or 64 when T*k >= 32*E;
                          // the shared expert's chunks (expert E) come last
  int32_t* meta;          // [0]: active routed experts, [1]: chunks, [2]: T*k; [32]: arrivals of the top-k + sort kernel
  int32_t* sort_wc;       // [64][E] per-wave expert counts, then bases (the many-assignment sort)
  int32_t* asg;           // [T*k + ns*T] assignments grouped by expert (shared: T*k + t, last)
  uint16_t* h16;          // [T*k + ns*T][f] w_j silu(g) u per position, fp16 operand order
  float* obuf;            // [T*k + ns*T][d] o_{t,j} per assignment
  // single-launch step (T = 1)
  unsigned long long* tagged_logits;  // ceil(E/4) lines of 128 B: (epoch << 32 | logit bits)
  unsigned long long* hrec;           // [k*f/8][5] (epoch << 32 | fp16 slice word)
  unsigned* epoch;                    // [kMaxFusedGrid] calls completed, per workgroup
  unsigned* error;                    // [1]  bit 0/1: a bounded wait timed out
};

constexpr int kMaxFusedGrid = 1024;
constexpr int kPhaseSlots = 16;  // phase timestamps per workgroup (diagnostic build, layer_kernel.h)
#ifdef MOE_PHASE_TRACE
// Copies the n first phase timestamps of the last int4 single-launch call
// ([workgroup][kPhaseSlots] 100 MHz counter values) to host memory.
hipError_t phase_trace_copy(unsigned long long* host, size_t n);
#endif
constexpr int kFusedGridCUs = 256;  // compute units the single-launch kernel is sized for (MI355X)
constexpr int kMaxGroupedGrid = 512;  // expert kernels: 2 resident workgroups on each of 256 CUs
constexpr int kMaxAssignments = MOE_MAX_TOKENS * MOE_MAX_TOPK;  // largest T*k

// Arguments of the single-launch 1-token layer kernel.
struct FusedArgs {
  const float* router_w;
  const float* router_b;
  const uint8_t* gate_q;
  const uint16_t* gate_s;
  const uint8_t* up_q;
  const uint16_t* up_s;
  const uint8_t* down_q;
  const uint16_t* down_s;
  const uint16_t* x;     // [d] bf16 (unused when resid_in is set)
  float* y;              // [d], or NULL in a stack
  const float* resid_in; // stack: fp32 residual r_l [d]; x = bf16(r / rms(r)); NULL otherwise
  float* resid_out;      // stack: r_{l+1} = r_l + y (a different buffer from resid_in)
  float eps;
  uint16_t* x_trace;     // stack: x_l [d], or NULL
  int32_t* idx_out;      // [k] or NULL
  float* w_out;          // [k] or NULL
  unsigned long long* logits;  // tagged logits, 4 per 128-byte line
  unsigned long long* hrec;    // tagged fp16 slices of h
  unsigned* epoch;             // per-workgroup call counts
  unsigned* error;
  unsigned long long* rrec;    // persistent stack: tagged r_l + y words for the next layer
  const uint8_t* sh_gate_q;    // the shared expert (ns = 1): slot k of the step, weight 1
  const uint16_t* sh_gate_s;
  const uint8_t* sh_up_q;
  const uint16_t* sh_up_s;
  const uint8_t* sh_down_q;
  const uint16_t* sh_down_s;
  const float* gate_tscale;  // NVFP4: fp32 scale of each expert matrix [E] (shared: [1])
  const float* up_tscale;
  const float* down_tscale;
  const float* sh_gate_tscale;
  const float* sh_up_tscale;
  const float* sh_down_tscale;
  int E, k, norm, ns;
  int fmt;  // expert weights: 0 int4, 1 MXFP4 (E8M0 bytes per 32), 2 NVFP4 (E4M3 bytes per 16 + gate_ts ...)
  unsigned spin_limit;  // polls of a bounded wait before it gives up (>= 1)
  unsigned tag_skew;    // 0; 1 makes every wait look for a tag no workgroup writes (tests of the error path)
};

constexpr unsigned kSpinLimit = 1u << 21;  // default polls of a bounded wait (about 2 s)

// Arguments of the persistent stack kernel: up to kMaxStackLayers layers of
// one shape per launch, each layer's FusedArgs read from the copy in its
// workspace (its per-call fields unused).
constexpr int kMaxStackLayers = 64;
struct StackArgs {
  const FusedArgs* layer[kMaxStackLayers];
  int L;
  const float* resid_in;   // r_0 [d]
  float* resid_out;        // r_L [d] (may be resid_in)
  float eps;
  uint16_t* x_trace;       // [L][d] or NULL
  float* y_trace;          // [L][d] or NULL
  int32_t* idx_trace;      // [L][k] or NULL
  unsigned spin_limit, tag_skew;
};
// The shape every layer of a persistent launch shares.
struct StackShape {
  int d, f, E, k, ns, fmt;
};

// The whole 1-token step in one launch, for the shapes it is built for
// (d, f) in {(256, 128), (2048, 512)}, E <= 256; ns shared experts take
// slots k .. k+ns-1.
bool fused_layer_supported(int d, int f, int E, int k, int ns, int G);
int fused_grid();
hipError_t launch_layer_fused(const FusedArgs& a, int d, int f, hipStream_t s);
// the per-format instances (grid G), in their own translation units
hipError_t launch_layer_int4(const FusedArgs& a, int d, int f, int G, hipStream_t s);
hipError_t launch_layer_mxfp4(const FusedArgs& a, int d, int f, int G, hipStream_t s);
hipError_t launch_layer_nvfp4(const FusedArgs& a, int d, int f, int G, hipStream_t s);
// The persistent stack kernel (grid G, the same as the single-launch kernel).
hipError_t launch_stack_fused(const StackArgs& a, const StackShape& sh, hipStream_t s);
hipError_t launch_stack_int4(const StackArgs& a, const StackShape& sh, int G, hipStream_t s);
hipError_t launch_stack_mxfp4(const StackArgs& a, const StackShape& sh, int G, hipStream_t s);
hipError_t launch_stack_nvfp4(const StackArgs& a, const StackShape& sh, int G, hipStream_t s);

// Router logits of T tokens (a matrix product), then softmax + top-k of
// every token and the assignments grouped by expert.  Activations come
// either from x (bf16 [T][d]) or, when x is NULL, from the fp32 residual
// r [T][d] normalized by RMSNorm (eps), written to x_trace when it is
// non-NULL (else to the workspace).
hipError_t launch_router(const LayerArgs& a, const uint16_t* x, const float* r, float eps, int T,
                         int32_t* idx_out, float* w_out, uint16_t* x_trace, hipStream_t s);

// Slices of K the router splits its sum into for T tokens, and the floats
// of its partial sums (logits workspace).
int router_splits(int T, int E, int d);
size_t router_partial_floats(int T, int E, int d);

// Per chosen expert, over all its tokens: h = w_j * silu(W_g x) * (W_u x).
hipError_t launch_gateup(const LayerArgs& a, int T, hipStream_t s);

// Per chosen expert, over all its tokens: o_{t,j} = W_d h; then
// y_t = sum_j o_{t,j} (+ o_{t,shared}) into y_out (if non-NULL) and
// residual_t += y_t (if non-NULL), inside the same kernel for small T.
hipError_t launch_down_combine(const LayerArgs& a, int T, float* y_out, float* residual, hipStream_t s);

// The tile-major copies of gate, up and down (from the canonical matrices)
// and the router's bf16 terms.
hipError_t launch_tile_weights(const LayerArgs& a, hipStream_t s);


// LM head GEMV + argmax.
hipError_t launch_lmhead(const uint8_t* wq, const uint16_t* ws, int V, int d, const uint16_t* x, int B,
                         int32_t* token, float* max_logit, void* workspace, hipStream_t s);

size_t lmhead_workspace_bytes(int V, int d, int B);

// The LM head with the library's own per-device scratch array as workspace
// (no allocation; calls overlapping on one GPU race); its size.
hipError_t launch_lmhead_noalloc(const uint8_t* wq, const uint16_t* ws, int V, int d, const uint16_t* x, int B,
                                 int32_t* token, float* max_logit, hipStream_t s);
size_t lmhead_scratch_bytes();

}  // namespace moe
