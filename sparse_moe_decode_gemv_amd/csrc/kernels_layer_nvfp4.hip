// kernels_layer_nvfp4.hip -- the single-launch 1-token layer step with
// NVFP4 (E2M1 codes, E4M3 scale per 16, fp32 per matrix) expert weights: the instances of layer_kernel.h for this format.
#include "layer_kernel.h"

namespace moe {

hipError_t launch_layer_nvfp4(const FusedArgs& a, int d, int f, int G, hipStream_t s) {
  return launch_layer_format<2>(a, d, f, G, s);
}

}  // namespace moe
