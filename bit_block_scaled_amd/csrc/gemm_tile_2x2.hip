// NVFP4 GEMM kernels of the 128x128 workgroup tile (wave tile 64x64),
// with and without a K tail and GELU; the kernel is in gemm_kernel.h.
#include "gemm_kernel.h"

namespace nvfp4 {

hipError_t launch_gemm_2x2(const GemmArgs &a, hipStream_t stream, int cus) {
  return launch_tile<2, 2>(a, stream, cus);
}

}  // namespace nvfp4
