// NVFP4 GEMM kernels of the 192x256 workgroup tile (wave tile 96x128),
// with and without a K tail and GELU; the kernel is in gemm_kernel.h.
#include "gemm_kernel.h"

namespace nvfp4 {

hipError_t launch_gemm_3x4(const GemmArgs &a, hipStream_t stream, int cus) {
  return launch_tile<3, 4>(a, stream, cus);
}

}  // namespace nvfp4
