// Internal helpers shared by the HIP sources of libgptstep (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace gs {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bit patterns in uint16_t)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16 with the hardware converter (v_cvt_pk_bf16_f32: round to
// nearest, ties to even; NaN stays NaN)
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f2bf(float f) {
  const __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  const bf16x2_hw v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// wave64 reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Non-temporal vector stores (data written once and read by a later kernel)
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_nt(void* p, uint4 w) {
  const u32x4_nt v = {w.x, w.y, w.z, w.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_nt*>(p));
}
__device__ __forceinline__ void st_nt(void* p, uint2 w) {
  const u32x2_nt v = {w.x, w.y};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2_nt*>(p));
}
__device__ __forceinline__ void st_nt(float* p, float4 f) {
  const f32x4_nt v = {f.x, f.y, f.z, f.w};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_nt*>(p));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// XCD-aware remap of a linear workgroup id.  The dispatcher places workgroup
// i on XCD i % 8; this returns an id such that each XCD sees one contiguous
// range of logical ids (so neighbouring tiles share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  const int q = nblk / 8, r = nblk % 8;
  const int xcd = bid % 8, loc = bid / 8;
  return (xcd < r) ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc;
}

}  // namespace gs

// ---------------------------------------------------------------------------
// host-side error plumbing (api.cpp owns the thread-local message)
// ---------------------------------------------------------------------------
namespace gs {
void set_error(const std::string& msg);
}

#define GS_HIP_CHECK(expr)                                                       \
  do {                                                                           \
    hipError_t e_ = (expr);                                                      \
    if (e_ != hipSuccess) {                                                      \
      gs::set_error(std::string(#expr) + ": " + hipGetErrorString(e_));          \
      return -4;                                                                 \
    }                                                                            \
  } while (0)

#define GS_LAUNCH_CHECK(name)                                                    \
  do {                                                                           \
    hipError_t e_ = hipGetLastError();                                           \
    if (e_ != hipSuccess) {                                                      \
      gs::set_error(std::string("launch of ") + name + ": " + hipGetErrorString(e_)); \
      return -4;                                                                 \
    }                                                                            \
  } while (0)
