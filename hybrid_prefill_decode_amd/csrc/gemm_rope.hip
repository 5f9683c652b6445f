// Token-batched GEMM kernels with the RoPE + KV append (QKV projection) epilogue, one instantiation per tile shape
// (the kernels themselves are in gemm_core.h).
#include "gemm_core.h"

namespace hl {

hipError_t launch_gemm_rope(const TileChoice& tc, const hl_bf16* a, const hl_bf16* w, hl_bf16* c,
                            int m, int n, int k, const GemmEpi& epi, float* part, hipStream_t st) {
  const TileChoice one{tc.bm, tc.bn, false, tc.splits, tc.tail};
  return epi.head_dim == 128
             ? launch_choice<kEpiRopeAppend, 128>(one, a, w, c, m, n, k, epi, part, st)
             : launch_choice<kEpiRopeAppend, 64>(one, a, w, c, m, n, k, epi, part, st);
}

}  // namespace hl
