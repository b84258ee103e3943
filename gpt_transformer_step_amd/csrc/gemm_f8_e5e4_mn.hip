// fp8 GEMM instantiations with m/n-contiguous operands, A E5M2 (output
// gradient), B E4M3: the data gradient dX = dY W reads the weight codes as
// stored (B n-contiguous), the weight gradient dW = dY^T X reads both
// operands' codes as stored (A m-contiguous, B n-contiguous), so neither
// needs transposed copies.
#include "gemm_kernel.h"

namespace gs {

int gemm_fp8_e5e4_mn(const GemmArgs& a, int epi, hipStream_t s) {
  if (a.a_kcontig && !a.b_kcontig) {
    switch (epi) {
      case EPI_F32: return launch_tiles<true, false, EPI_F32, 2>(a, s);
      case EPI_BF16: return launch_tiles<true, false, EPI_BF16, 2>(a, s);
      case EPI_DRELU2: return launch_tiles<true, false, EPI_DRELU2, 2>(a, s);
      default: break;
    }
  } else if (!a.a_kcontig && !a.b_kcontig && epi == EPI_F32) {
    return launch_tiles<false, false, EPI_F32, 2>(a, s);
  }
  set_error("gemm_fp8: epilogue or operand layouts not built for E5M2 x E4M3");
  return -5;
}

}  // namespace gs
