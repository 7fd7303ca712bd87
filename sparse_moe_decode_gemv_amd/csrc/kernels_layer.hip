// kernels_layer.hip -- host side of the single-launch 1-token layer step:
// which shapes it takes, its grid, and the dispatch to the per-format
// instances (the kernel itself is in layer_kernel.h; int4 is instantiated
// here, MXFP4 and NVFP4 in their own files).
#include "layer_kernel.h"

namespace moe {

// Work each wave takes in the fused kernel must fit one unit per wave; k
// counts the expert slots (chosen plus shared).
static bool fits(int d, int f, int E, int k, int G) {
  const int W = 4 * G;
  if (k > 16) return false;
  const int cpr = d / 32, cprf = f / 32;
  if ((long)k * f * cpr / 256 > W) return false;  // gate/up units (4 pieces per lane)
  int kp = 1;
  while (kp < k) kp <<= 1;
  const int P = kp * cprf;
  const int lprd = P > 64 ? P / 64 : 1, rpld = P < 64 ? 64 / P : 1;
  const int nld = lprd > 4 ? lprd : 4;
  const int rows_w = (nld / lprd) * rpld;
  if (d / rows_w > W) return false;
  if ((size_t)kp * (f / 8) * 5 * sizeof(unsigned) > 64 * 1024) return false;  // slices of h in LDS
  if (E > 256 || E > W) return false;
  return true;
}

bool fused_layer_supported(int d, int f, int E, int k, int ns, int G) {
  if (!((d == 256 && f == 128) || (d == 2048 && f == 512))) return false;
  return fits(d, f, E, k + ns, G);
}

int fused_grid() {
  static int g = 0;
  if (!g) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 0;
    g = cus > kMaxFusedGrid ? kMaxFusedGrid : cus;
  }
  return g;
}

hipError_t launch_layer_int4(const FusedArgs& a, int d, int f, int G, hipStream_t s) {
  return launch_layer_format<0>(a, d, f, G, s);
}

hipError_t launch_stack_int4(const StackArgs& a, const StackShape& sh, int G, hipStream_t s) {
  return launch_stack_format<0>(a, sh, G, s);
}

hipError_t launch_stack_fused(const StackArgs& a, const StackShape& sh, hipStream_t s) {
  const int G = fused_grid();
  if (G <= 0 || a.L < 1 || a.L > kMaxStackLayers || !fits(sh.d, sh.f, sh.E, sh.k + sh.ns, G)) return hipErrorInvalidValue;
  if (sh.fmt == 2) return launch_stack_nvfp4(a, sh, G, s);
  if (sh.fmt == 1) return launch_stack_mxfp4(a, sh, G, s);
  return launch_stack_int4(a, sh, G, s);
}

#ifdef MOE_PHASE_TRACE
hipError_t phase_trace_copy(unsigned long long* host, size_t n) {
  if (n > (size_t)kMaxFusedGrid * kPhaseSlots) n = (size_t)kMaxFusedGrid * kPhaseSlots;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_ts), n * sizeof(unsigned long long), 0, hipMemcpyDeviceToHost);
}
#endif

hipError_t launch_layer_fused(const FusedArgs& a, int d, int f, hipStream_t s) {
  const int G = fused_grid();
  if (G <= 0 || !fits(d, f, a.E, a.k + a.ns, G)) return hipErrorInvalidValue;
  if (a.fmt == 2) return launch_layer_nvfp4(a, d, f, G, s);
  if (a.fmt == 1) return launch_layer_mxfp4(a, d, f, G, s);
  return launch_layer_int4(a, d, f, G, s);
}

}  // namespace moe
