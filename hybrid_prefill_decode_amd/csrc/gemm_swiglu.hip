// Token-batched GEMM kernels with the SwiGLU epilogue, one instantiation per tile shape
// (the kernels themselves are in gemm_core.h).
#include "gemm_core.h"

namespace hl {

hipError_t launch_gemm_swiglu(const TileChoice& tc, const hl_bf16* a, const hl_bf16* w, hl_bf16* c,
                              int m, int n, int k, const GemmEpi& epi, float* part,
                              hipStream_t st) {
  return launch_choice<HL_EPI_SWIGLU>(TileChoice{tc.bm, tc.bn, false, tc.splits, tc.tail}, a, w, c, m, n,
                                      k, epi, part, st);
}

}  // namespace hl
