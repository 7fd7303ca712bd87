/*
 * moe_decode.h -- C ABI of the sparse MoE decode library for MI355X (gfx950).
 *
 * One decode step of a 4-bit mixture-of-experts layer (router GEMV, softmax
 * and top-k expert choice, int4 gate/up GEMVs over the chosen experts only,
 * SwiGLU, int4 down GEMV, weighted combine), a pre-norm stack of such layers,
 * and the 4-bit output layer (LM head) GEMV with a fused argmax.
 *
 * The pages describe the model these calls serve: every MoE layer holds 256
 * routed experts of which a small router picks a few per token, and the
 * output layer, about an eighth of the per-token work, is stored in 4 bits
 * ("Flint 40B: Best Mid Sized LLM", transcript 02:35-05:39).  The unit of
 * work follows their statement of the problem, decode speed in tokens per
 * second: one call advances T tokens through one layer, or B hidden rows
 * through the LM head.
 *
 * Conventions for every call:
 *   - Pointers marked (device) point to GPU memory that the caller allocated
 *     and owns; the library never allocates, frees or copies device memory
 *     except the one-time workspace clear in moe_decode_init.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     device work is enqueued on it and the call returns without waiting.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and no output is touched.  Faults inside a
 *     kernel surface at the caller's next synchronization.
 *   - No C++ exception crosses this interface.
 *
 * Stored int4 weight format (all int4 matrices: experts and LM head):
 *   A matrix [rows][K] (K a power of two, >= 128) takes K/2 bytes per row,
 *   rows one after another.  Element k of a row is held in byte
 *   64*t + 16*q + 4*j + e/2 of the row, with t = k/128, j = (k%128)/32,
 *   q = (k%32)/8, e = k%8; the low nibble for even e, the high nibble for
 *   odd e.  The nibble is a code u in 0..15 and the weight is
 *   (u - 8) * scale[row][k/32], scale an IEEE binary16 bit pattern stored
 *   row-major [rows][K/32].  (Each 16-byte piece of a row thus holds 8
 *   elements of each of 4 consecutive groups of 32.)
 *   The pages list 4-bit integer builds among the releases and a 4-bit output
 *   layer but give no group size or layout; this format is the library's.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;

#define MOE_OK 0
#define MOE_ERR_NULL (-1)        /* a required pointer is NULL */
#define MOE_ERR_SHAPE (-2)       /* a size is out of range or inconsistent */
#define MOE_ERR_ALIGN (-3)       /* a device pointer is not 16-byte aligned */
#define MOE_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required */
#define MOE_ERR_HIP (-5)         /* the HIP runtime refused a launch or copy */
#define MOE_ERR_UNSUPPORTED (-6) /* a shape the kernels are not built for */

#define MOE_MAX_TOPK 16          /* largest top_k */
#define MOE_MAX_TOKENS 4096      /* largest T per forward call (prompt processing included) */
#define MOE_LMHEAD_MAX_B 16      /* largest B per LM-head call */

/* Shape of one MoE layer.
 *   d          hidden width, a power of two in [256, 8192]
 *   f          expert FFN width, a power of two in [128, 4096]
 *   n_experts  E, routed experts, in [1, 1024]
 *   top_k      k, experts chosen per token, in [1, min(E, MOE_MAX_TOPK)]
 *   norm_topk  1: the chosen softmax weights are divided by their sum;
 *              0: they are used as they are
 *   max_tokens largest T a forward call will pass, in [1, MOE_MAX_TOKENS]
 *   n_shared   0, or 1 for an always-on shared expert of the routed experts'
 *              shape whose output is added with weight 1 (the pages' layer
 *              has six routed experts plus one shared, "Flint 40B: Best Mid
 *              Sized LLM", transcript 02:35); it takes no part in the
 *              softmax or the renormalization
 *   weight_format  MOE_WEIGHTS_INT4, MOE_WEIGHTS_MXFP4 or MOE_WEIGHTS_NVFP4
 *              (the pages name NVFP4 as the released model's format,
 *              "Recursive Releases Flint...", section "Quantization").  Both
 *              FP4 formats hold FP4 E2M1 codes at the int4 nibble positions.
 *              MXFP4: one E8M0 scale byte 2^(b-127) per 32 elements (OCP MX
 *              v1.0; byte 255, NaN, is not supported; the batched kernels,
 *              which round each weight to fp16, are exact for bytes
 *              104..140: moe_decode_init scans the scale bytes and returns
 *              MOE_ERR_UNSUPPORTED for a 255, or for a byte outside
 *              104..140 in a layer that may run the batched kernels).  NVFP4: one FP8 E4M3 scale byte per 16 elements
 *              (OCP E4M3FN) and one fp32 scale per expert matrix
 *              (moe_layer_weights.*_tscale) */
#define MOE_WEIGHTS_INT4 0
#define MOE_WEIGHTS_MXFP4 1
#define MOE_WEIGHTS_NVFP4 2
typedef struct {
  int32_t d, f, n_experts, top_k, norm_topk, max_tokens, n_shared;
  int32_t weight_format;
} moe_layer_desc;

/* Weights of one MoE layer (device, read-only, owned by the caller, must
 * outlive the handle; every pointer 16-byte aligned).
 *   router_w  fp32 [E][d] row-major
 *   router_b  fp32 [E], or NULL for no bias
 *   gate_q    int4 [E][f][d/2] stored format, gate_s binary16 [E][f][d/32]
 *   up_q      int4 [E][f][d/2],                up_s   binary16 [E][f][d/32]
 *   down_q    int4 [E][d][f/2],                down_s binary16 [E][d][f/32]
 *   with weight_format MOE_WEIGHTS_MXFP4 each *_q holds E2M1 codes and each
 *             *_s points to E8M0 bytes [...][K/32] (same shapes, one byte
 *             per scale; pass the byte array's address in the field);
 *             with MOE_WEIGHTS_NVFP4 each *_s points to E4M3 bytes
 *             [...][K/16] and gate_tscale, up_tscale, down_tscale are fp32
 *             [E] (shared_*_tscale fp32 [1]), 4-byte aligned; they are
 *             ignored (may be NULL) for the other formats
 *   shared_*  the shared expert's matrices in the same formats without the
 *             expert dimension ([f][d/2], [f][d/32], [d][f/2], [d][f/32]);
 *             required when n_shared = 1, ignored (may be NULL) otherwise */
typedef struct {
  const float* router_w;
  const float* router_b;
  const uint8_t* gate_q;
  const uint16_t* gate_s;
  const uint8_t* up_q;
  const uint16_t* up_s;
  const uint8_t* down_q;
  const uint16_t* down_s;
  const uint8_t* shared_gate_q;
  const uint16_t* shared_gate_s;
  const uint8_t* shared_up_q;
  const uint16_t* shared_up_s;
  const uint8_t* shared_down_q;
  const uint16_t* shared_down_s;
  const float* gate_tscale;
  const float* up_tscale;
  const float* down_tscale;
  const float* shared_gate_tscale;
  const float* shared_up_tscale;
  const float* shared_down_tscale;
} moe_layer_weights;

typedef struct moe_layer* moe_handle;

/* Bytes of device workspace a layer with this shape needs (0 on a bad
 * shape).  The workspace holds the router's partial sums (at most about
 * max(4*T*E bytes, 8 MiB)), the chosen experts, their grouping by expert,
 * the operand copies of the activations, the SwiGLU activations and the
 * per-assignment expert outputs of one call (for max_tokens T: about
 * T*k*(4d + 2f) + 8Td bytes, plus 32*E + 10*k*f bytes of single-launch
 * hand-off words and 6 KiB) and, for a
 * layer that may run the batched kernels (max_tokens > 1, or a shape the
 * single-launch kernel does not take), a tile-major copy of the gate, up and
 * down matrices, the shared expert's included (their size: 3*(E+n_shared)*
 * d*f/2 bytes of codes + 3*(E+n_shared)*d*f/16 of scales, twice that for
 * NVFP4, whose copy holds binary16 block scales with the matrix scale folded
 * in), and the router
 * matrix as three bfloat16 terms whose sum is exactly W_r (6*E*d bytes, E
 * rounded up to 16). */
size_t moe_decode_workspace_bytes(const moe_layer_desc* desc);

/* Validate the shape and weights and bind them, with a caller-owned device
 * workspace of at least moe_decode_workspace_bytes(desc) bytes, into a host
 * handle.  Clears the workspace once and, when the layer may run the
 * batched kernels, writes the tile-major copy of the expert matrices and
 * the router's bf16 terms (synchronously, on the null stream); batched
 * calls read those copies, so router or expert weights changed after init
 * reach only the single-launch 1-token step.  The handle owns no device memory.  One handle must not run on two streams
 * at once (its workspace is shared by its calls); distinct handles are
 * independent. */
moe_status moe_decode_init(const moe_layer_desc* desc, const moe_layer_weights* weights,
                           void* workspace, size_t workspace_bytes, moe_handle* out);

/* The same as moe_decode_init, with its device work (the workspace clear, the
 * MXFP4 scale scan, the batched path's copies, the persistent stack's
 * argument copy) enqueued on `stream` (hipStream_t; NULL = the null stream),
 * and only that stream synchronized before it returns: the init of the
 * boundary as stated for this library, taking the caller's stream like every
 * other call.  It synchronizes, so it must not be called while `stream` is
 * being captured into a graph.  Same validation, errors and ownership as
 * moe_decode_init. */
moe_status moe_decode_init_on_stream(const moe_layer_desc* desc, const moe_layer_weights* weights,
                                     void* workspace, size_t workspace_bytes, void* stream, moe_handle* out);

/* One decode step of T tokens through the layer (per token a router picks a
 * few of the routed experts and only those run, "Flint 40B: Best Mid Sized
 * LLM", transcript 02:35):
 *   logits = W_r x_t + b;  p = softmax(logits) over all E experts;
 *   S = the k largest p (larger first, lower expert index on ties);
 *   w_j = p_j / sum_{i in S} p_i (norm_topk) or p_j;
 *   y_t = sum_{j in S} w_j * W_d[j] (silu(W_g[j] x_t) * (W_u[j] x_t))
 *         [+ W_d^s (silu(W_g^s x_t) * (W_u^s x_t)) with a shared expert].
 * Only the chosen experts' (and the shared expert's) weights are read.
 *   x         (device) bf16 bit patterns [T][d]
 *   T         tokens, 1 <= T <= max_tokens
 *   y         (device) fp32 [T][d], overwritten
 *   topk_idx  (device) int32 [T][k], chosen experts in the order above, or NULL
 *   topk_w    (device) fp32 [T][k], their weights, or NULL (routed experts
 *             only: the shared expert's weight is always 1)
 * T = 1 on a shape the single-launch kernel is built for ((d, f) = (256,
 * 128) or (2048, 512), E <= 256, k + n_shared <= 16) runs as one launch of
 * one workgroup per compute unit that hands data between its phases through
 * memory; it needs all of its workgroups resident at once.  Its waits are
 * bounded: if other work on the GPU keeps some workgroups from starting
 * until a wait gives up, the call still ends but its outputs are not valid,
 * and moe_decode_error_flags reports it.
 * Intermediate precision: the router, gate/up and down sums accumulate in
 * fp32.  The SwiGLU activations reach the down projection in binary16
 * (relative rounding 2^-11) as h 2^(2a), with 2^a the power of two that
 * puts the token's largest |x| in [1, 2) and the output scaled back by
 * 2^(-2a): exact scalings, so x of any magnitude works; what must stay
 * below 65504 is w_j silu(g) u computed from x 2^a, which the weights
 * bound (at most about 4 |W_g row|_1 |W_u row|_1), and elements of h 2^(2a)
 * below 2^-14 keep fewer bits.  The batched kernels (T > 1) also round each
 * dequantized weight q*s and each element of x 2^a to binary16 (elements
 * below 2^-14 of the token's largest lose low bits). */
moe_status moe_decode_forward(moe_handle h, const uint16_t* x, int32_t T, float* y,
                              int32_t* topk_idx, float* topk_w, void* stream);

/* L layers in sequence on a residual stream, each pre-normed by an RMSNorm
 * of unit weight (the attention blocks between MoE layers are not part of
 * this call):
 *   x_l = bf16_rne(r_l / sqrt(mean(r_l^2) + eps));  r_{l+1} = r_l + layer_l(x_l).
 * Each layer runs as forward would run it for T tokens (one launch at T = 1
 * where its shape allows, else the batched kernels), so layers of different
 * shapes and max_tokens may be mixed.
 *   layers    L handles of equal d and top_k, each with its own workspace
 *   residual  (device) fp32 [T][d], r_0 in, r_L out
 *   x_trace   (device) bf16 [L][T][d] receiving every x_l, or NULL
 *   y_trace   (device) fp32 [L][T][d] receiving every layer output, or NULL
 *   idx_trace (device) int32 [L][T][k] receiving every chosen set, or NULL */
moe_status moe_decode_stack_forward(const moe_handle* layers, int32_t L, float* residual, int32_t T,
                                    float eps, uint16_t* x_trace, float* y_trace, int32_t* idx_trace,
                                    void* stream);

/* moe_decode_stack_forward with options.
 *   flags  0: as moe_decode_stack_forward (one launch, or the batched
 *          kernels, per layer);
 *          MOE_STACK_PERSISTENT: at T = 1, a run of layers that all take the
 *          single-launch kernel with the same shape (d, f, top_k, n_shared,
 *          weight_format, and E in the same band: <= 64, <= 128 or <= 256)
 *          runs as one persistent launch per 64 layers: every workgroup
 *          steps through the layers in turn, each layer's output reaching
 *          the next as tagged words in the workspace, and the next layer's
 *          router rows loading while the current layer's SwiGLU activations
 *          are exchanged (the pages' decode kernel fuses the whole pass into
 *          one launch, "Flint 40B: Best Mid Sized LLM", transcript 06:43).
 *          Layers it does not apply to run as without the flag.
 * The result is the same either way, bit for bit.  (On MI355X the hand-off
 * of the 8 KB residual between all workgroups costs about as much as the
 * kernel boundary it replaces, so the persistent launch is not faster per
 * layer; it takes one launch instead of L.) */
#define MOE_STACK_PERSISTENT 1
moe_status moe_decode_stack_forward_ex(const moe_handle* layers, int32_t L, float* residual, int32_t T,
                                       float eps, uint16_t* x_trace, float* y_trace, int32_t* idx_trace,
                                       int32_t flags, void* stream);

/* The grouping of (token, slot) assignments to routed experts made by the handle's
 * last forward or stack call that ran the batched kernels (T > 1, or a
 * shape without the single-launch kernel).  Assignment a = t*k + j is
 * token t's j-th chosen expert.  Copies, enqueued on `stream` (any output
 * may be NULL):
 *   offsets     (device) int32 [E+1]: expert e owns positions
 *               offsets[e] .. offsets[e+1]-1; offsets[E] = T*k
 *   assignments (device) int32 [T*k]: the assignments ordered by expert,
 *               ascending a within an expert
 *   active      (device) int32 [E]: the experts with at least one
 *               assignment, ascending (entries past n_active undefined)
 *   n_active    (device) int32 [1]
 * T must be the token count of that call.  The batched step reads each
 * chosen expert's weights once for all its tokens in this order. */
moe_status moe_decode_expert_groups(moe_handle h, int32_t T, int32_t* offsets, int32_t* assignments,
                                    int32_t* active, int32_t* n_active, void* stream);

/* Flags the layer's single-launch kernel raised since they were last
 * cleared: bit 0, a wait for the other workgroups' router logits gave up;
 * bit 1, a wait for the SwiGLU activations gave up; bit 2 (persistent
 * stack), a wait for the previous layer's output gave up.  Any means that
 * the call's outputs are not valid (see moe_decode_forward).  Enqueues on
 * `stream` a copy of the flags to `flags` (device uint32 [1], or NULL) and,
 * when clear != 0, resets them, so the copy is ordered after every call
 * enqueued before it on that stream. */
moe_status moe_decode_error_flags(moe_handle h, uint32_t* flags, int32_t clear, void* stream);

/* Diagnostic setting of the single-launch kernel's bounded waits, for tests
 * of the error path: each wait gives up after `polls` rounds (>= 1; the
 * default, restored by passing 1u << 21, is about 2 s), and with
 * unreachable = 1 every wait looks for a tag no workgroup writes, so every
 * wait gives up and the call ends with both flags set.  Host-side only; it
 * applies to calls enqueued afterwards. */
moe_status moe_decode_set_wait_limit(moe_handle h, uint32_t polls, int32_t unreachable);

/* Repack int4 (or FP4) codes from the canonical order -- element k of a row
 * in byte k/2, the low nibble for even k, rows of K/2 bytes one after
 * another -- into the stored format above (the scales keep their layout).
 * Enqueued on `stream`.
 *   src, dst  (device) [rows][K/2] bytes each, 16-byte aligned, not
 *             overlapping (MOE_ERR_SHAPE if they do)
 *   rows      >= 1;  K  a multiple of 128 */
moe_status moe_int4_repack(const uint8_t* src, uint8_t* dst, int64_t rows, int32_t K, void* stream);

/* Diagnostic for measurements: reads `bytes` (a multiple of 16) from the
 * device buffer `buf` with 16-byte loads spread over every compute unit
 * (sixteen workgroups of 256 threads per CU, each reading a contiguous
 * range, eight loads in flight per thread) and writes nothing but, in
 * practice never, one word to `sink` (device uint32 [1]).  Timing it over a buffer larger than
 * the memory-side cache gives the read bandwidth a plain streaming kernel
 * achieves on this GPU, the "achievable" figure beside the 8 TB/s peak. */
moe_status moe_decode_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Diagnostic for measurements: the phase timestamps of the last int4
 * single-launch layer call (one token through one layer, the chain of
 * phases -- router, logit exchange, top-k, gate/up, h exchange, down -- of
 * "Flint 40B: Best Mid Sized LLM", transcript 02:35, in one kernel).
 * Recorded only by the library built with MOE_PHASE_TRACE
 * (`python -m sparse_moe_decode_gemv_amd.build --phase-trace`, a separate
 * libmoe_decode_phase.so); every other build returns MOE_ERR_UNSUPPORTED.
 * Copies min(n, 1024 * 16) values [workgroup][16] of the GPU's 100 MHz
 * real-time counter, written by thread 0 of each workgroup at 11 marked
 * points (slots 0..10; slot 2 by the router workgroups only).  Synchronous:
 * the caller synchronizes the stream of that call first.
 *   host_out  (host) uint64 [n] */
moe_status moe_decode_phase_trace(uint64_t* host_out, int64_t n);

/* Free the host handle (no device memory is touched). NULL is ignored. */
void moe_decode_destroy(moe_handle h);

/* Bytes of device workspace lmhead_int4_argmax needs for this shape (0 on a
 * bad shape). */
size_t lmhead_int4_argmax_workspace_bytes(int32_t V, int32_t d, int32_t B);

/* 4-bit output layer with greedy decoding ("Flint 40B: Best Mid Sized LLM",
 * transcript 03:36-05:39; mirrorspeed.com page, section "Quantization"):
 *   z[b][v] = sum_k W[v][k] x[b][k];  token[b] = the smallest v with the
 *   largest z[b][v];  max_logit[b] = that z (fp32).
 * The logits are never written to memory.
 *   w_q, w_s  (device) int4 [V][d/2] stored format and binary16 [V][d/32]
 *   V         vocabulary rows, 1 <= V <= 2^24
 *   d         hidden width, a power of two in [256, 8192]
 *   x         (device) bf16 [B][d]
 *   B         rows, 1 <= B <= MOE_LMHEAD_MAX_B
 *   token     (device) int32 [B]
 *   max_logit (device) fp32 [B], or NULL
 *   workspace (device) at least lmhead_int4_argmax_workspace_bytes(V, d, B)
 *             bytes, 256-byte aligned, zero-filled before its first use:
 *             it holds arrival counters, which every call leaves at zero
 *             again, and per-workgroup partial results, which need no
 *             clearing.  Calls sharing a workspace must not overlap. */
moe_status lmhead_int4_argmax(const uint8_t* w_q, const uint16_t* w_s, int32_t V, int32_t d,
                              const uint16_t* x, int32_t B, int32_t* token, float* max_logit,
                              void* workspace, size_t workspace_bytes, void* stream);

/* The same as lmhead_int4_argmax, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): no workspace argument.  The library keeps a fixed
 * scratch array of 557,568 bytes on each GPU it runs on (the workspace of
 * the largest B), held until the process ends; the first call on a device
 * takes its address and enqueues a clear of its counters.  Calls with a
 * shape whose workspace would exceed it return MOE_ERR_WORKSPACE (none of
 * the shapes accepted above does).  All calls on one GPU share the array:
 * calls that overlap in time on one GPU (other streams, other threads)
 * race and must be serialized by the caller.  Nothing is allocated or
 * freed, by the library or through any library it calls. */
moe_status lmhead_int4_argmax_noalloc(const uint8_t* w_q, const uint16_t* w_s, int32_t V, int32_t d,
                                      const uint16_t* x, int32_t B, int32_t* token, float* max_logit, void* stream);

/* Text for a status code (static storage). */
const char* moe_status_str(moe_status s);

/* Version of this interface (incremented on incompatible changes). */
int32_t moe_decode_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
