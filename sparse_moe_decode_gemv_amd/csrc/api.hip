// api.hip -- the C ABI (include/moe_decode.h): validation, workspace layout
// and kernel dispatch.  All checks run on the host before anything is
// enqueued; no C++ exception leaves this file.
#include <hip/hip_runtime.h>

#include <new>

#include "moe_decode.h"
#include "launch.h"

namespace {

constexpr int kAbiVersion = 4;

struct Layout {
  size_t logits, sel_idx, sel_w, xp, xn, off, act, chunk_off, chunks, asg, h16, obuf, resid, tagged,
      hrec, epoch, sort_wc, cleared;             // [0, cleared) is zeroed at init
  size_t gate_t, gate_ts, up_t, up_ts, down_t, down_ts;  // tile-major expert copies (0 bytes if unused)
  size_t router_t;                                       // bf16 terms of the router matrix (same)
  size_t total;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

moe_status check_desc(const moe_layer_desc* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->d < 1 || d->f < 1 || d->n_experts < 1 || d->top_k < 1 || d->max_tokens < 1) return MOE_ERR_SHAPE;
  if (d->top_k > d->n_experts || d->top_k > MOE_MAX_TOPK) return MOE_ERR_SHAPE;
  if (d->max_tokens > MOE_MAX_TOKENS || d->n_experts > 1024) return MOE_ERR_SHAPE;
  if (d->norm_topk != 0 && d->norm_topk != 1) return MOE_ERR_SHAPE;
  if (d->n_shared != 0 && d->n_shared != 1) return MOE_ERR_SHAPE;
  if (d->weight_format != MOE_WEIGHTS_INT4 && d->weight_format != MOE_WEIGHTS_MXFP4 &&
      d->weight_format != MOE_WEIGHTS_NVFP4)
    return MOE_ERR_SHAPE;
  if (d->d % 32 || d->f % 32) return MOE_ERR_SHAPE;
  if (!is_pow2(d->d) || d->d < 256 || d->d > 8192) return MOE_ERR_UNSUPPORTED;
  if (!is_pow2(d->f) || d->f < 128 || d->f > 4096) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The batched kernels read a tile-major copy of the expert matrices, made
// at init; a layer gets one if it may run them: T > 1 allowed, or a shape
// without the single-launch kernel (which reads the caller's matrices).
bool needs_tiled_copy(const moe_layer_desc* d) {
  return d->max_tokens > 1 ||
         !moe::fused_layer_supported(d->d, d->f, d->n_experts, d->top_k, d->n_shared, moe::kFusedGridCUs);
}

Layout layout_of(const moe_layer_desc* d) {
  Layout L;
  const size_t T = (size_t)d->max_tokens, E = (size_t)d->n_experts, k = (size_t)d->top_k;
  const size_t ns = (size_t)d->n_shared;
  size_t o = 0;
  const size_t Tk = T * k, d_ = (size_t)d->d, f_ = (size_t)d->f;
  const size_t Ta = Tk + ns * T;  // assignments, the shared expert's last
  size_t part = 0;  // router partial sums: the most any T <= max_tokens needs
  for (int t = 1; t <= d->max_tokens; ++t) {
    const size_t n = moe::router_partial_floats(t, d->n_experts, d->d);
    part = n > part ? n : part;
  }
  L.logits = o, o += align256(part * sizeof(float));
  L.sel_idx = o, o += align256(Tk * sizeof(int32_t));
  L.sel_w = o, o += align256(Tk * sizeof(float));
  L.xp = o, o += align256(T * d_ * sizeof(uint16_t));
  L.xn = o, o += align256(T * d_ * sizeof(uint16_t));
  L.off = o, o += align256((E + 1 + 4) * sizeof(int32_t));  // off[E+1], then meta
  L.act = o, o += align256(E * sizeof(int32_t));
  L.chunk_off = o, o += align256((E + 1) * sizeof(int32_t));
  L.chunks = o, o += align256(((E < Tk ? E : Tk) + Tk / 32 + ns * ((T + 31) / 32)) * 4 * sizeof(int32_t));
  L.asg = o, o += align256(Ta * sizeof(int32_t));
  L.h16 = o, o += align256(Ta * f_ * sizeof(uint16_t));
  L.obuf = o, o += align256(Ta * d_ * sizeof(float));
  L.resid = o, o += align256(T * d_ * sizeof(float));  // second residual buffer of a stack
  L.tagged = o, o += align256((E + 3) / 4 * 128);                          // 4 logits per line
  L.hrec = o, o += align256((k + ns) * (size_t)(d->f / 8) * 5 * sizeof(unsigned long long) * 2);  // + line padding
  L.epoch = o, o += align256((size_t)(moe::kMaxFusedGrid + 1) * sizeof(unsigned));  // epochs, error
  L.sort_wc = o, o += align256(T > 1 ? (size_t)64 * E * sizeof(int32_t) : 0);      // per-wave counts of the wide sort
  L.cleared = o;
  const bool copy = needs_tiled_copy(d);
  // scale copy: 2 bytes per 32 elements (int4, MXFP4 uses half), 4 for NVFP4 (fp16 per 16 elements)
  const size_t sb = d->weight_format == MOE_WEIGHTS_NVFP4 ? 4 : 2;
  const size_t cq = copy ? (E + ns) * f_ * d_ / 2 : 0, cs = copy ? (E + ns) * f_ * (d_ / 32) * sb : 0;
  L.gate_t = o, o += align256(cq);
  L.gate_ts = o, o += align256(cs);
  L.up_t = o, o += align256(cq);
  L.up_ts = o, o += align256(cs);
  L.down_t = o, o += align256(cq);  // E*d*f/2 bytes as well
  L.down_ts = o, o += align256(cs);
  L.router_t = o, o += align256(copy ? (E + 15) / 16 * 16 * d_ * 3 * sizeof(uint16_t) : 0);
  L.total = o;
  return L;
}

}  // namespace

struct moe_layer {
  moe_layer_desc desc;
  moe::LayerArgs args;
  void* workspace;
  float* resid_tmp;  // [max_tokens][d]: the other residual buffer when this layer leads a stack
  bool fused;        // the 1-token step runs as one launch
};

namespace {

moe::FusedArgs fused_args(const moe_layer* h) {
  const moe::LayerArgs& a = h->args;
  moe::FusedArgs f{};
  f.router_w = a.router_w, f.router_b = a.router_b;
  f.gate_q = a.gate_q, f.gate_s = a.gate_s, f.up_q = a.up_q, f.up_s = a.up_s;
  f.down_q = a.down_q, f.down_s = a.down_s;
  f.logits = a.tagged_logits, f.hrec = a.hrec, f.epoch = a.epoch, f.error = a.error;
  f.sh_gate_q = a.sh_gate_q, f.sh_gate_s = a.sh_gate_s, f.sh_up_q = a.sh_up_q, f.sh_up_s = a.sh_up_s;
  f.sh_down_q = a.sh_down_q, f.sh_down_s = a.sh_down_s;
  f.E = a.E, f.k = a.k, f.norm = a.norm_topk, f.ns = a.ns;
  f.fmt = a.fmt;
  f.gate_tscale = a.gate_tscale, f.up_tscale = a.up_tscale, f.down_tscale = a.down_tscale;
  f.sh_gate_tscale = a.sh_gate_tscale, f.sh_up_tscale = a.sh_up_tscale, f.sh_down_tscale = a.sh_down_tscale;
  return f;
}

}  // namespace

extern "C" {

int32_t moe_decode_abi_version(void) { return kAbiVersion; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MOE_ERR_ALIGN: return "a device pointer is not suitably aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "the HIP runtime reported an error";
    case MOE_ERR_UNSUPPORTED: return "shape not supported by the kernels";
    default: return "unknown status";
  }
}

size_t moe_decode_workspace_bytes(const moe_layer_desc* desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  return layout_of(desc).total;
}

moe_status moe_decode_init(const moe_layer_desc* desc, const moe_layer_weights* w, void* workspace,
                           size_t workspace_bytes, moe_handle* out) {
  if (!out) return MOE_ERR_NULL;
  *out = nullptr;
  const moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (!w || !w->router_w || !w->gate_q || !w->gate_s || !w->up_q || !w->up_s || !w->down_q || !w->down_s)
    return MOE_ERR_NULL;
  const void* ptrs[] = {w->router_w, w->gate_q, w->gate_s, w->up_q, w->up_s, w->down_q, w->down_s};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  if (w->router_b && !aligned4(w->router_b)) return MOE_ERR_ALIGN;
  if (desc->n_shared) {
    if (!w->shared_gate_q || !w->shared_gate_s || !w->shared_up_q || !w->shared_up_s || !w->shared_down_q ||
        !w->shared_down_s)
      return MOE_ERR_NULL;
    const void* sp[] = {w->shared_gate_q, w->shared_gate_s, w->shared_up_q, w->shared_up_s, w->shared_down_q,
                        w->shared_down_s};
    for (const void* p : sp)
      if (!aligned16(p)) return MOE_ERR_ALIGN;
  }
  if (desc->weight_format == MOE_WEIGHTS_NVFP4) {  // the matrices' fp32 scales
    if (!w->gate_tscale || !w->up_tscale || !w->down_tscale) return MOE_ERR_NULL;
    if (desc->n_shared && (!w->shared_gate_tscale || !w->shared_up_tscale || !w->shared_down_tscale))
      return MOE_ERR_NULL;
    const void* tp[] = {w->gate_tscale, w->up_tscale, w->down_tscale, w->shared_gate_tscale, w->shared_up_tscale,
                        w->shared_down_tscale};
    for (const void* p : tp)
      if (p && !aligned4(p)) return MOE_ERR_ALIGN;
  }
  const Layout L = layout_of(desc);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return MOE_ERR_ALIGN;

  moe_layer* h = new (std::nothrow) moe_layer;
  if (!h) return MOE_ERR_HIP;
  h->desc = *desc;
  h->workspace = workspace;
  moe::LayerArgs& a = h->args;
  a.d = desc->d, a.f = desc->f, a.E = desc->n_experts, a.k = desc->top_k, a.norm_topk = desc->norm_topk;
  a.ns = desc->n_shared;
  a.fmt = desc->weight_format;
  a.gate_tscale = w->gate_tscale, a.up_tscale = w->up_tscale, a.down_tscale = w->down_tscale;
  a.sh_gate_tscale = w->shared_gate_tscale, a.sh_up_tscale = w->shared_up_tscale;
  a.sh_down_tscale = w->shared_down_tscale;
  a.router_w = w->router_w, a.router_b = w->router_b;
  a.gate_q = w->gate_q, a.gate_s = w->gate_s, a.up_q = w->up_q, a.up_s = w->up_s;
  a.down_q = w->down_q, a.down_s = w->down_s;
  a.sh_gate_q = a.ns ? w->shared_gate_q : nullptr, a.sh_gate_s = a.ns ? w->shared_gate_s : nullptr;
  a.sh_up_q = a.ns ? w->shared_up_q : nullptr, a.sh_up_s = a.ns ? w->shared_up_s : nullptr;
  a.sh_down_q = a.ns ? w->shared_down_q : nullptr, a.sh_down_s = a.ns ? w->shared_down_s : nullptr;
  unsigned char* base = static_cast<unsigned char*>(workspace);
  a.logits = reinterpret_cast<float*>(base + L.logits);
  a.sel_idx = reinterpret_cast<int32_t*>(base + L.sel_idx);
  a.sel_w = reinterpret_cast<float*>(base + L.sel_w);
  a.xp = reinterpret_cast<uint16_t*>(base + L.xp);
  a.xn = reinterpret_cast<uint16_t*>(base + L.xn);
  a.sort_wc = reinterpret_cast<int32_t*>(base + L.sort_wc);
  a.off = reinterpret_cast<int32_t*>(base + L.off);
  a.meta = a.off + desc->n_experts + 1;
  a.act = reinterpret_cast<int32_t*>(base + L.act);
  a.chunk_off = reinterpret_cast<int32_t*>(base + L.chunk_off);
  a.chunks = reinterpret_cast<int4*>(base + L.chunks);
  a.asg = reinterpret_cast<int32_t*>(base + L.asg);
  a.h16 = reinterpret_cast<uint16_t*>(base + L.h16);
  a.obuf = reinterpret_cast<float*>(base + L.obuf);
  h->resid_tmp = reinterpret_cast<float*>(base + L.resid);
  a.tagged_logits = reinterpret_cast<unsigned long long*>(base + L.tagged);
  a.hrec = reinterpret_cast<unsigned long long*>(base + L.hrec);
  a.epoch = reinterpret_cast<unsigned*>(base + L.epoch);
  a.error = a.epoch + moe::kMaxFusedGrid;
  const bool copy = needs_tiled_copy(desc);
  a.gate_t = copy ? base + L.gate_t : nullptr;
  a.gate_ts = copy ? reinterpret_cast<uint16_t*>(base + L.gate_ts) : nullptr;
  a.up_t = copy ? base + L.up_t : nullptr;
  a.up_ts = copy ? reinterpret_cast<uint16_t*>(base + L.up_ts) : nullptr;
  a.down_t = copy ? base + L.down_t : nullptr;
  a.down_ts = copy ? reinterpret_cast<uint16_t*>(base + L.down_ts) : nullptr;
  a.router_t = copy ? reinterpret_cast<uint16_t*>(base + L.router_t) : nullptr;
  h->fused = moe::fused_layer_supported(desc->d, desc->f, desc->n_experts, desc->top_k, desc->n_shared,
                                        moe::fused_grid());
  if (!h->fused && !copy) {  // a GPU with fewer CUs than the single-launch kernel assumes
    delete h;
    return MOE_ERR_UNSUPPORTED;
  }
  if (hipMemset(workspace, 0, L.cleared) != hipSuccess || (copy && moe::launch_tile_weights(a, nullptr) != hipSuccess) ||
      hipDeviceSynchronize() != hipSuccess) {
    delete h;
    return MOE_ERR_HIP;
  }
  *out = h;
  return MOE_OK;
}

void moe_decode_destroy(moe_handle h) { delete h; }

moe_status moe_decode_expert_groups(moe_handle h, int32_t T, int32_t* offsets, int32_t* assignments,
                                    int32_t* active, int32_t* n_active, void* stream) {
  if (!h) return MOE_ERR_NULL;
  if (T < 1 || T > h->desc.max_tokens) return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe::LayerArgs& a = h->args;
  const size_t E = (size_t)a.E, Tk = (size_t)T * a.k;
  struct {
    void* dst;
    const void* src;
    size_t n;
  } cp[] = {{offsets, a.off, (E + 1) * 4}, {assignments, a.asg, Tk * 4}, {active, a.act, E * 4},
            {n_active, a.meta, 4}};
  for (const auto& c : cp)
    if (c.dst && hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDeviceToDevice, s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_decode_forward(moe_handle h, const uint16_t* x, int32_t T, float* y, int32_t* topk_idx,
                              float* topk_w, void* stream) {
  if (!h || !x || !y) return MOE_ERR_NULL;
  if (T < 1 || T > h->desc.max_tokens) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(y)) return MOE_ERR_ALIGN;
  if ((topk_idx && !aligned4(topk_idx)) || (topk_w && !aligned4(topk_w))) return MOE_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe::LayerArgs& a = h->args;
  if (T == 1 && h->fused) {
    moe::FusedArgs f = fused_args(h);
    f.x = x, f.y = y, f.idx_out = topk_idx, f.w_out = topk_w;
    return moe::launch_layer_fused(f, a.d, a.f, s) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  if (moe::launch_router(a, x, nullptr, 0.f, T, topk_idx, topk_w, nullptr, s) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_gateup(a, T, s) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_down(a, T, s) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_combine(a, T, y, nullptr, s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_decode_stack_forward(const moe_handle* layers, int32_t L, float* residual, int32_t T, float eps,
                                    uint16_t* x_trace, float* y_trace, int32_t* idx_trace, void* stream) {
  if (!layers || !residual) return MOE_ERR_NULL;
  if (L < 1 || T < 1) return MOE_ERR_SHAPE;
  if (!(eps >= 0.f)) return MOE_ERR_SHAPE;
  for (int l = 0; l < L; ++l) {
    if (!layers[l]) return MOE_ERR_NULL;
    if (layers[l]->desc.d != layers[0]->desc.d || layers[l]->desc.top_k != layers[0]->desc.top_k)
      return MOE_ERR_SHAPE;
    if (T > layers[l]->desc.max_tokens) return MOE_ERR_SHAPE;
  }
  if (!aligned16(residual) || (x_trace && !aligned16(x_trace)) || (y_trace && !aligned16(y_trace)) ||
      (idx_trace && !aligned4(idx_trace)))
    return MOE_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t d = (size_t)layers[0]->desc.d, k = (size_t)layers[0]->desc.top_k;
  bool fused = T == 1;
  for (int l = 0; l < L; ++l) fused = fused && layers[l]->fused;
  if (fused) {
    // One launch per layer.  The residual alternates between the caller's
    // buffer and the first layer's spare one, arranged so that r_L lands in
    // the caller's buffer, except for odd L, which ends with one copy.
    float* buf[2] = {residual, layers[0]->resid_tmp};
    for (int l = 0; l < L; ++l) {
      moe::FusedArgs f = fused_args(layers[l]);
      f.resid_in = buf[l & 1];
      f.resid_out = buf[(l + 1) & 1];
      f.eps = eps;
      f.y = y_trace ? y_trace + (size_t)l * d : nullptr;
      f.x_trace = x_trace ? x_trace + (size_t)l * d : nullptr;
      f.idx_out = idx_trace ? idx_trace + (size_t)l * k : nullptr;
      if (moe::launch_layer_fused(f, layers[l]->args.d, layers[l]->args.f, s) != hipSuccess) return MOE_ERR_HIP;
    }
    if ((L & 1) && hipMemcpyAsync(residual, buf[1], d * sizeof(float), hipMemcpyDeviceToDevice, s) != hipSuccess)
      return MOE_ERR_HIP;
    return MOE_OK;
  }
  for (int l = 0; l < L; ++l) {
    const moe::LayerArgs& a = layers[l]->args;
    uint16_t* xt = x_trace ? x_trace + (size_t)l * T * d : nullptr;
    int32_t* it = idx_trace ? idx_trace + (size_t)l * T * k : nullptr;
    float* yt = y_trace ? y_trace + (size_t)l * T * d : nullptr;
    if (moe::launch_router(a, nullptr, residual, eps, T, it, nullptr, xt, s) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_gateup(a, T, s) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_down(a, T, s) != hipSuccess) return MOE_ERR_HIP;
    if (moe::launch_combine(a, T, yt, residual, s) != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

size_t lmhead_int4_argmax_workspace_bytes(int32_t V, int32_t d, int32_t B) {
  if (V < 1 || V > (1 << 24) || !is_pow2(d) || d < 256 || d > 8192 || B < 1 || B > MOE_LMHEAD_MAX_B) return 0;
  return moe::lmhead_workspace_bytes(V, d, B);
}

moe_status lmhead_int4_argmax(const uint8_t* w_q, const uint16_t* w_s, int32_t V, int32_t d, const uint16_t* x,
                              int32_t B, int32_t* token, float* max_logit, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!w_q || !w_s || !x || !token) return MOE_ERR_NULL;
  if (V < 1 || V > (1 << 24) || B < 1 || B > MOE_LMHEAD_MAX_B || d < 1 || d % 32) return MOE_ERR_SHAPE;
  if (!is_pow2(d) || d < 256 || d > 8192) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(w_q) || !aligned16(w_s) || !aligned16(x) || !aligned4(token) ||
      (max_logit && !aligned4(max_logit)))
    return MOE_ERR_ALIGN;
  if (!workspace || workspace_bytes < moe::lmhead_workspace_bytes(V, d, B)) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return MOE_ERR_ALIGN;
  if (moe::launch_lmhead(w_q, w_s, V, d, x, B, token, max_logit, workspace, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

}  // extern "C"
