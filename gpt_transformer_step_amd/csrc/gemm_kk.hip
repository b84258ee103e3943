// Instantiations of the bf16 GEMM kernel for one operand layout
// (A k-contiguous, B k-contiguous).
#include "gemm_kernel.h"

namespace gs {

int gemm_bf16_kk(const GemmArgs& a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_F32: return launch_tiles<true, true, EPI_F32>(a, s);
    case EPI_BF16: return launch_tiles<true, true, EPI_BF16>(a, s);
    case EPI_RESID: return launch_tiles<true, true, EPI_RESID>(a, s);
    case EPI_RELU2: return launch_tiles<true, true, EPI_RELU2>(a, s);
    case EPI_CE_FWD: return launch_tiles<true, true, EPI_CE_FWD>(a, s);
    case EPI_QKV: return launch_tiles<true, true, EPI_QKV>(a, s);
    default:
      set_error("gemm_bf16: epilogue not built for this operand layout");
      return -5;
  }
}

}  // namespace gs
