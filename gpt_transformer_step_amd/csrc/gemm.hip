// Dispatch of the bf16 GEMM family by operand layout (kernel in gemm_kernel.h).
#include "gemm_kernel.h"

namespace gs {

int gemm_bf16_kk(const GemmArgs& a, int epi, hipStream_t s);
int gemm_bf16_km(const GemmArgs& a, int epi, hipStream_t s);
int gemm_bf16_mm(const GemmArgs& a, int epi, hipStream_t s);
int gemm_bf16_mk(const GemmArgs& a, int epi, hipStream_t s);

int gemm_tile_n(const GemmArgs& a) { return use_big_tile(a) ? 256 : 128; }

long long gemm_amax_slots(const GemmArgs& a) {
  const bool big = use_big_tile(a);
  const int t = big ? 256 : 128;
  const long long tiles = (long long)((a.M + t - 1) / t) * ((a.N + t - 1) / t);
  return tiles * a.batch * a.k_split * (big ? Cfg<256, 256>::NT : Cfg<128, 128>::NT) / 64;
}

int gemm_bf16(const GemmArgs& a, int epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return 0;
  // the cross-entropy epilogue takes the row max on the unscaled products
  if (epi == EPI_CE_FWD && !(a.alpha > 0.f)) {
    set_error("gemm: the cross-entropy epilogue needs alpha > 0");
    return -1;
  }
  if (a.a_kcontig && a.b_kcontig) return gemm_bf16_kk(a, epi, s);
  if (a.a_kcontig) return gemm_bf16_km(a, epi, s);
  if (a.b_kcontig) return gemm_bf16_mk(a, epi, s);
  return gemm_bf16_mm(a, epi, s);
}

}  // namespace gs
