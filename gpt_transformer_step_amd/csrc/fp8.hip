// Per-tensor fp8 quantisation for the fp8 block products (apidog.com/pt
// "Gerenciamento de Precisão" and apidog.com/de "Präzisionsverwaltung": most
// linear layers in fp8 with one scale per tensor).
//
//   amax  = max |x| over the whole tensor          (amax_partial + fp8_scale)
//   s     = fmax / amax in fp32 (1 when amax == 0)  fmax: 448 (E4M3), 57344 (E5M2)
//   code  = RNE(clamp(x * s, -fmax, fmax))          (fp8_quant)
//
// The hardware converter (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32, OCP formats on
// gfx950) rounds to nearest even but does not saturate, so values are clamped
// to +-fmax first.  The quantiser writes the codes in the tensor's layout,
// transposed, or both: fp8 products take both operands k-contiguous, so the
// data-gradient product needs W^T and the weight-gradient product needs
// dY^T and X^T.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gs {

namespace {

__device__ __forceinline__ float fmax_of(int fmt) { return fmt ? 57344.f : 448.f; }

template <bool F32>
__device__ __forceinline__ void load4(const void* x, long long idx, float* v) {
  if constexpr (F32) {
    const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + idx);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + idx);
    v[0] = lo_bf(w.x); v[1] = hi_bf(w.x); v[2] = lo_bf(w.y); v[3] = hi_bf(w.y);
  }
}

// max |x| over rows x cols, one partial per block.  Contiguous tensors
// (ld == cols; cols % 16 == 0) are read as a flat array, 64 bytes per thread
// per round (four independent 16-byte loads in flight); others row by row.
template <bool F32>
__device__ __forceinline__ float amax16(const void* x, long long idx) {
  // 16 bytes at element idx: 8 bf16 or 4 fp32
  if constexpr (F32) {
    const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + idx);
    return fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w)));
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + idx);
    // |bf16| compares like its bit pattern with the sign cleared
    const uint32_t m = 0x7fff7fffu;
    const uint32_t a = max(max((w.x & m) & 0xffffu, (w.x & m) >> 16), max((w.y & m) & 0xffffu, (w.y & m) >> 16));
    const uint32_t b = max(max((w.z & m) & 0xffffu, (w.z & m) >> 16), max((w.w & m) & 0xffffu, (w.w & m) >> 16));
    return bf2f((uint16_t)max(a, b));
  }
}

// Batched over blockIdx.y: tensor b starts sx elements after tensor b - 1 and
// writes its partials gridDim.x floats after b - 1's.
template <bool F32>
__global__ void __launch_bounds__(256) amax_partial_kernel(const void* __restrict__ xv, long long ldx, int rows,
                                                          int cols, float* __restrict__ partial, long long sx) {
  constexpr int EPC = F32 ? 4 : 8;  // elements per 16 bytes
  const void* x = reinterpret_cast<const char*>(xv) + (long long)blockIdx.y * sx * (F32 ? 4 : 2);
  partial += (long long)blockIdx.y * gridDim.x;
  float m = 0.f;
  if (ldx == cols) {
    const long long n16 = (long long)rows * cols / EPC;
    const long long stride = (long long)gridDim.x * 256;
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
      const float a0 = amax16<F32>(x, i * EPC), a1 = amax16<F32>(x, (i + stride) * EPC);
      const float a2 = amax16<F32>(x, (i + 2 * stride) * EPC), a3 = amax16<F32>(x, (i + 3 * stride) * EPC);
      m = fmaxf(m, fmaxf(fmaxf(a0, a1), fmaxf(a2, a3)));
    }
    for (; i < n16; i += stride) m = fmaxf(m, amax16<F32>(x, i * EPC));
  } else {
    // rows * cols / 4 < 2^31 (checked on the host): 32-bit index arithmetic
    const unsigned c4 = (unsigned)cols / 4u;
    const unsigned n4 = (unsigned)rows * c4;
    for (unsigned i = blockIdx.x * 256u + threadIdx.x; i < n4; i += gridDim.x * 256u) {
      const unsigned r = i / c4, c = (i - r * c4) * 4u;
      float v[4];
      load4<F32>(x, (long long)r * ldx + c, v);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    }
  }
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One workgroup of 1024 threads: the partial maxima (up to a few tens of
// thousands) are read with eight independent loads in flight per thread, so
// the reduction costs a few load latencies rather than one per 256 values.
constexpr int kScaleNT = 1024;
// (batched: workgroup b reduces partials b np .. and writes scale[b sstride])
__global__ void __launch_bounds__(kScaleNT) fp8_scale_kernel(const float* __restrict__ partial, long long np,
                                                            int fmt, float* __restrict__ scale, long long sstride) {
  partial += (long long)blockIdx.x * np;
  scale += (long long)blockIdx.x * sstride;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  long long i = threadIdx.x;
  for (; i + 7 * kScaleNT < np; i += 8 * kScaleNT) {
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = fmaxf(m[u], partial[i + u * kScaleNT]);
  }
  for (; i < np; i += kScaleNT) m[0] = fmaxf(m[0], partial[i]);
  float mm = fmaxf(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])), fmaxf(fmaxf(m[4], m[5]), fmaxf(m[6], m[7])));
  mm = wave_max(mm);
  __shared__ float red[kScaleNT / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mm;
  __syncthreads();
  if (threadIdx.x == 0) {
    float amax = 0.f;
#pragma unroll
    for (int w = 0; w < kScaleNT / 64; ++w) amax = fmaxf(amax, red[w]);
    scale[0] = amax > 0.f ? fmax_of(fmt) / amax : 1.f;
  }
}

// two fp8 codes (low 16 bits of the result)
template <int FMT>
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  if constexpr (FMT == 0) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
  else return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false) & 0xffffu;
}

// 128 x 128 tile per block; thread t owns the 8 x 8 block at rows 8 (t / 16),
// columns 8 (t % 16): 16-byte loads (a wave covers four 256-byte row
// segments), 8-byte code stores, and the transposed codes through LDS,
// written as 16-byte row chunks.  rows % 16 == 0 and cols % 16 == 0, so
// every 8-row or 8-column block lies wholly inside or outside the tensor.
constexpr int kQT2 = 128;
constexpr int kLDT2 = kQT2 + 8;  // LDS row (bytes) of the transposed tile, padded against bank conflicts

template <bool F32>
__device__ __forceinline__ void load8(const void* x, long long idx, float* v) {
  if constexpr (F32) {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + idx);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + idx + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + idx);
    v[0] = lo_bf(w.x); v[1] = hi_bf(w.x); v[2] = lo_bf(w.y); v[3] = hi_bf(w.y);
    v[4] = lo_bf(w.z); v[5] = hi_bf(w.z); v[6] = lo_bf(w.w); v[7] = hi_bf(w.w);
  }
}

// Batched over blockIdx.z with element strides sx (x), ss (scale), sq (q, qt).
template <bool F32, int FMT>
__global__ void __launch_bounds__(256) fp8_quant128_kernel(const void* __restrict__ xv, long long ldx, int rows,
                                                          int cols, const float* __restrict__ scale,
                                                          uint8_t* __restrict__ q, long long ldq,
                                                          uint8_t* __restrict__ qt, long long ldqt, long long sx,
                                                          long long ss, long long sq) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kQT2 * kLDT2];
  const int bz = blockIdx.z;
  const void* x = reinterpret_cast<const char*>(xv) + (long long)bz * sx * (F32 ? 4 : 2);
  scale += (long long)bz * ss;
  if (q) q += (long long)bz * sq;
  if (qt) qt += (long long)bz * sq;
  const int t = threadIdx.x;
  const int r0 = blockIdx.y * kQT2, c0 = blockIdx.x * kQT2;
  const int rb = 8 * (t >> 4), cb = 8 * (t & 15);
  const float s = scale[0];
  const float fm = fmax_of(FMT);
  const bool in = (r0 + rb < rows) && (c0 + cb < cols);
  uint2 rw[8];  // codes of row i, columns 0..7
  if (in) {
    float v[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) load8<F32>(x, (long long)(r0 + rb + i) * ldx + c0 + cb, v[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = fminf(fmaxf(v[i][j] * s, -fm), fm);
      rw[i] = make_uint2(cvt2<FMT>(v[i][0], v[i][1]) | (cvt2<FMT>(v[i][2], v[i][3]) << 16),
                         cvt2<FMT>(v[i][4], v[i][5]) | (cvt2<FMT>(v[i][6], v[i][7]) << 16));
    }
    if (q) {
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<uint2*>(q + (long long)(r0 + rb + i) * ldq + c0 + cb) = rw[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) rw[i] = make_uint2(0u, 0u);
  }
  if (!qt) return;  // launch-uniform
  // column j of the 8 x 8 block (rows rb .. rb+7) into row cb + j of the transposed tile
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wi = j < 4 ? rw[i].x : rw[i].y, wj = j < 4 ? rw[i + 4].x : rw[i + 4].y;
      lo |= ((wi >> (8 * (j & 3))) & 0xffu) << (8 * i);
      hi |= ((wj >> (8 * (j & 3))) & 0xffu) << (8 * i);
    }
    *reinterpret_cast<uint2*>(tile + (cb + j) * kLDT2 + rb) = make_uint2(lo, hi);
  }
  __syncthreads();
  // row c of the transposed tile = column c0 + c of x: 128 codes in 8 chunks of 16
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = t + 256 * k;
    const int c = idx >> 3, seg = 16 * (idx & 7);
    if (c0 + c < cols && r0 + seg < rows) {
      const uint2* src = reinterpret_cast<const uint2*>(tile + c * kLDT2 + seg);
      const uint2 a = src[0], b = src[1];
      *reinterpret_cast<uint4*>(qt + (long long)(c0 + c) * ldqt + r0 + seg) = make_uint4(a.x, a.y, b.x, b.y);
    }
  }
}

}  // namespace

int fp8_partials(long long rows, long long cols) {
  const long long n4 = rows * cols / 4;
  return (int)std::max<long long>(1, std::min<long long>(kFp8Partials, (n4 + 255) / 256));
}

int launch_fp8_amax_scale(const void* x, int is_f32, long long ldx, int rows, int cols, int fmt, float* partial,
                          float* scale, hipStream_t s, int count, long long sx, long long sscale) {
  const int np = fp8_partials(rows, cols);
  if (count <= 0) return 0;
  if (is_f32)
    hipLaunchKernelGGL(amax_partial_kernel<true>, dim3(np, count), dim3(256), 0, s, x, ldx, rows, cols, partial, sx);
  else
    hipLaunchKernelGGL(amax_partial_kernel<false>, dim3(np, count), dim3(256), 0, s, x, ldx, rows, cols, partial, sx);
  GS_LAUNCH_CHECK("amax_partial");
  hipLaunchKernelGGL(fp8_scale_kernel, dim3(count), dim3(kScaleNT), 0, s, partial, (long long)np, fmt, scale, sscale);
  GS_LAUNCH_CHECK("fp8_scale");
  return 0;
}

int launch_fp8_quant(const void* x, int is_f32, long long ldx, int rows, int cols, int fmt, const float* scale,
                     uint8_t* q, long long ldq, uint8_t* qt, long long ldqt, hipStream_t s, int count, long long sx,
                     long long sscale, long long sq) {
  if (rows <= 0 || cols <= 0 || count <= 0) return 0;
  dim3 grid((cols + kQT2 - 1) / kQT2, (rows + kQT2 - 1) / kQT2, count);
#define GS_Q(F, M) hipLaunchKernelGGL((fp8_quant128_kernel<F, M>), grid, dim3(256), 0, s, x, ldx, rows, cols, scale, q, ldq, qt, ldqt, sx, sscale, sq)
  if (is_f32) {
    if (fmt) GS_Q(true, 1); else GS_Q(true, 0);
  } else {
    if (fmt) GS_Q(false, 1); else GS_Q(false, 0);
  }
#undef GS_Q
  GS_LAUNCH_CHECK("fp8_quant");
  return 0;
}

int quantize_fp8(const void* x, int is_f32, long long ldx, int rows, int cols, int fmt, float* partial, float* scale,
                 uint8_t* q, long long ldq, uint8_t* qt, long long ldqt, hipStream_t s) {
  int rc = launch_fp8_amax_scale(x, is_f32, ldx, rows, cols, fmt, partial, scale, s);
  if (rc) return rc;
  return launch_fp8_quant(x, is_f32, ldx, rows, cols, fmt, scale, q, ldq, qt, ldqt, s);
}

int quantize_fp8_partials(const void* x, int is_f32, long long ldx, int rows, int cols, int fmt,
                          const float* partial, long long np, float* scale, uint8_t* q, long long ldq, uint8_t* qt,
                          long long ldqt, hipStream_t s) {
  hipLaunchKernelGGL(fp8_scale_kernel, dim3(1), dim3(kScaleNT), 0, s, partial, np, fmt, scale, 0LL);
  GS_LAUNCH_CHECK("fp8_scale");
  return launch_fp8_quant(x, is_f32, ldx, rows, cols, fmt, scale, q, ldq, qt, ldqt, s);
}

}  // namespace gs
