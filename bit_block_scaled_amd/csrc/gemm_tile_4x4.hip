// NVFP4 GEMM kernels of the 256x256 workgroup tile (wave tile 128x128),
// with and without a K tail and GELU; the kernel is in gemm_kernel.h.
#include "gemm_kernel.h"

namespace nvfp4 {

hipError_t launch_gemm_4x4(const GemmArgs &a, hipStream_t stream, int cus) {
  return launch_tile<4, 4>(a, stream, cus);
}

}  // namespace nvfp4
