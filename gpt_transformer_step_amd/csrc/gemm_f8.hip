// fp8 GEMM dispatch.  Forward products are E4M3 x E4M3 with both operands
// k-contiguous (gemm_f8_e4e4.hip); data- and weight-gradient products are
// E5M2 (output gradient) x E4M3, k-contiguous (gemm_f8_e5e4.hip) or with the
// codes read as stored: B n-contiguous for the data gradient, both m/n-
// contiguous for the weight gradient (gemm_f8_e5e4_mn.hip).  The other two
// pairings exist with the plain fp32 epilogue, k-contiguous
// (gemm_f8_e4e5.hip, gemm_f8_e5e5.hip).  Each format pair is compiled in its
// own translation unit (the compiler's optimiser fails on one that holds the
// scaled fp8 MFMA with two different format pairs).
#include "common.h"
#include "gemm.h"

namespace gs {

int gemm_fp8_e4e4(const GemmArgs& a, int epi, hipStream_t s);
int gemm_fp8_e5e4(const GemmArgs& a, int epi, hipStream_t s);
int gemm_fp8_e4e5(const GemmArgs& a, int epi, hipStream_t s);
int gemm_fp8_e5e5(const GemmArgs& a, int epi, hipStream_t s);
int gemm_fp8_e5e4_mn(const GemmArgs& a, int epi, hipStream_t s);

int gemm_fp8(const GemmArgs& a, int epi, int fmt_a, int fmt_b, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return 0;
  if (!a.scale_a || !a.scale_b) {
    set_error("gemm_fp8: scale pointers are NULL");
    return -1;
  }
  if (!a.a_kcontig || !a.b_kcontig) {
    if (fmt_a != 1 || fmt_b != 0 || (!a.a_kcontig && a.b_kcontig)) {
      set_error("gemm_fp8: m/n-contiguous operands are built for E5M2 x E4M3 with B m/n-contiguous only");
      return -5;
    }
    // 16-byte chunks of codes along the contiguous dimension lie wholly
    // inside or outside the operand
    if ((!a.a_kcontig && a.M % 16) || (!a.b_kcontig && a.N % 16)) {
      set_error("gemm_fp8: an m/n-contiguous operand needs its rows (M or N) a multiple of 16");
      return -1;
    }
    return gemm_fp8_e5e4_mn(a, epi, s);
  }
  if (fmt_a == 0 && fmt_b == 0) return gemm_fp8_e4e4(a, epi, s);
  if (fmt_a == 1 && fmt_b == 0) return gemm_fp8_e5e4(a, epi, s);
  if (fmt_a == 0 && fmt_b == 1) return gemm_fp8_e4e5(a, epi, s);
  return gemm_fp8_e5e5(a, epi, s);
}

}  // namespace gs
