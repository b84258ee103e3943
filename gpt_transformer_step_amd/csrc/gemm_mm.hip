// Instantiations of the bf16 GEMM kernel for one operand layout
// (A mn-contiguous, B mn-contiguous).
#include "gemm_kernel.h"

namespace gs {

int gemm_bf16_mm(const GemmArgs& a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_F32: return launch_tiles<false, false, EPI_F32>(a, s);
    case EPI_BF16: return launch_tiles<false, false, EPI_BF16>(a, s);
    case EPI_F32_ATOMIC: return launch_tiles<false, false, EPI_F32_ATOMIC>(a, s);
    case EPI_F32_BF16: return launch_tiles<false, false, EPI_F32_BF16>(a, s);
    default:
      set_error("gemm_bf16: epilogue not built for this operand layout");
      return -5;
  }
}

}  // namespace gs
