// kernels_layer_mxfp4.hip -- the single-launch 1-token layer step with
// MXFP4 (E2M1 codes, E8M0 scale per 32) expert weights: the instances of layer_kernel.h for this format
// (one layer per launch, and the persistent stack).
#include "layer_kernel.h"

namespace moe {

hipError_t launch_layer_mxfp4(const FusedArgs& a, int d, int f, int G, hipStream_t s) {
  return launch_layer_format<1>(a, d, f, G, s);
}

hipError_t launch_stack_mxfp4(const StackArgs& a, const StackShape& sh, int G, hipStream_t s) {
  return launch_stack_format<1>(a, sh, G, s);
}

}  // namespace moe
