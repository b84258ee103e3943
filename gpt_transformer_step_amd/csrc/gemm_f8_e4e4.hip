// fp8 GEMM instantiations: A E4M3, B E4M3 (the forward block products).
#include "gemm_kernel.h"

namespace gs {

int gemm_fp8_e4e4(const GemmArgs& a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_F32: return launch_tiles<true, true, EPI_F32, 1>(a, s);
    case EPI_BF16: return launch_tiles<true, true, EPI_BF16, 1>(a, s);
    case EPI_RESID: return launch_tiles<true, true, EPI_RESID, 1>(a, s);
    case EPI_RELU2: return launch_tiles<true, true, EPI_RELU2, 1>(a, s);
    case EPI_QKV: return launch_tiles<true, true, EPI_QKV, 1>(a, s);
    default:
      set_error("gemm_fp8: epilogue not built for E4M3 x E4M3");
      return -5;
  }
}

}  // namespace gs
