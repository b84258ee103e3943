// fp8 GEMM instantiation: A E4M3, B E5M2, fp32 output.
#include "gemm_kernel.h"

namespace gs {

int gemm_fp8_e4e5(const GemmArgs& a, int epi, hipStream_t s) {
  if (epi == EPI_F32) return launch_tiles<true, true, EPI_F32, 3>(a, s);
  set_error("gemm_fp8: epilogue not built for E4M3 x E5M2");
  return -5;
}

}  // namespace gs
