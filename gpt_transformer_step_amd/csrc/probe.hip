// Roofline probes: an MFMA-only loop that measures the matrix-core rate the
// device sustains (no memory traffic), for the bf16 and fp8 instructions the
// step uses.  Each wave keeps 8 independent accumulators so the matrix pipe
// never waits on a dependency.

#include "common.h"
#include "kernels.h"

namespace gs {

namespace {

template <int FP8>
__global__ void __launch_bounds__(256) mfma_peak_kernel(int iters, float* out) {
  f32x16_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  const int lane = threadIdx.x & 63;
  if constexpr (FP8) {
    i32x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) { a[e] = 0x38383838 + lane + e; b[e] = 0x30303030 + e; }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i], 0, 0, 0, 127, 0, 127);
    }
  } else {
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) { a[e] = (short)(0x3f80 + lane); b[e] = (short)(0x3f80 + e); }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[i][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// flops per launch are returned in *flops: blocks * 4 waves * iters * 8 MFMAs * flops per MFMA
int launch_mfma_peak(int fp8, int blocks, int iters, float* out, double* flops, hipStream_t s) {
  if (fp8)
    hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(blocks), dim3(256), 0, s, iters, out);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(blocks), dim3(256), 0, s, iters, out);
  GS_LAUNCH_CHECK("mfma_peak");
  const double per = fp8 ? 32.0 * 32 * 64 * 2 : 32.0 * 32 * 16 * 2;
  *flops = (double)blocks * 4 * iters * 8 * per;
  return 0;
}

}  // namespace gs
