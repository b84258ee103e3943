// fp8 GEMM instantiations: A E5M2 (output gradient), B E4M3 (the data- and
// weight-gradient block products).
#include "gemm_kernel.h"

namespace gs {

int gemm_fp8_e5e4(const GemmArgs& a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_F32: return launch_tiles<true, true, EPI_F32, 2>(a, s);
    case EPI_BF16: return launch_tiles<true, true, EPI_BF16, 2>(a, s);
    case EPI_DRELU2: return launch_tiles<true, true, EPI_DRELU2, 2>(a, s);
    default:
      set_error("gemm_fp8: epilogue not built for E5M2 x E4M3");
      return -5;
  }
}

}  // namespace gs
