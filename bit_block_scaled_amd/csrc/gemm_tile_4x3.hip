// NVFP4 GEMM kernels of the 256x192 workgroup tile (wave tile 128x96),
// with and without a K tail and GELU; the kernel is in gemm_kernel.h.
#include "gemm_kernel.h"

namespace nvfp4 {

hipError_t launch_gemm_4x3(const GemmArgs &a, hipStream_t stream, int cus) {
  return launch_tile<4, 3>(a, stream, cus);
}

}  // namespace nvfp4
