// GEMM family on CDNA4 matrix cores: bf16 (v_mfma_f32_32x32x16_bf16) and
// fp8 (v_mfma_scale_f32_32x32x64_f8f6f4, OCP E4M3 / E5M2 codes).
//
// Every dense contraction of the step runs here: the q/k/v, output, MLP and
// head projections of the model passage (dev.to "¿Cómo Entrenar Tu Propio
// ChatGPT por $50?", "1. Modelo GPT"; the bf16 cast of weights in
// "3. Gestión de Precisión"), their data and weight gradients, the chunked
// head/cross-entropy products, the three products of each Newton-Schulz
// iteration ("2. Optimizador Muon": A = X^T X, B = b A + c A A, X = a X + X B),
// and the fp8 block products with one scale per tensor (apidog.com/pt
// "Gerenciamento de Precisão").
//
// Design (gfx950):
//   * 256x256 tiles with 8 waves (two per SIMD), or 128x128 tiles with 4; the
//     waves form a (waves/2) x 2 grid, each owning 64 rows and BN/2 columns.
//     One LDS stage holds 128 bytes of k per row (64 bf16 or 128 fp8 codes).
//   * Operands are staged in LDS, double buffered, one barrier per stage;
//     interior tiles are copied global -> LDS directly (global_load_lds), so
//     the next stage's loads are in flight while this stage's MFMAs run.
//   * Each operand tile sits in LDS in its memory layout.  A k-contiguous tile
//     is read as MFMA fragments with 16-byte loads; an m/n-contiguous bf16 tile
//     (the weight-gradient, data-gradient and Gram operands) is read with the
//     gfx950 transpose load ds_read_b64_tr_b16, two per fragment, so no bf16
//     product needs a transposed copy in HBM; an m/n-contiguous fp8 tile (the
//     data- and weight-gradient operands) with ds_read_b64_tr_b8, four per
//     fragment, so the quantiser writes each tensor's codes once.
//     Both layouts are XOR-swizzled so fragment reads are bank-conflict free
//     (64 banks of 4 bytes, 16-lane groups per 16-byte read).
//   * The MFMA is issued with the operands swapped (B tile as src0), so each
//     lane's accumulators hold one output row and groups of 4 consecutive
//     columns: stores are 8/16-byte vectors and row reductions (the
//     cross-entropy epilogue) stay inside a lane pair.
//   * Workgroup ids (over the whole grid: tiles x batch x k-splits) are
//     remapped so each of the 8 XCDs walks a contiguous range of the
//     (batch, split, tile) order, tiles rasterised in groups of 8 row tiles
//     for L2 reuse.

#pragma once

#include <type_traits>

#include "common.h"
#include "gemm.h"

namespace gs {
namespace {

// F8 template parameter: 0 = bf16 operands; 1 + fa + 2 fb = fp8 operands with
// A in format fa and B in format fb (0 = E4M3, 1 = E5M2).
constexpr int f8_fmt_a(int f8) { return (f8 - 1) & 1; }
constexpr int f8_fmt_b(int f8) { return (f8 - 1) >> 1; }
// K elements per LDS stage (128 bytes per row)
constexpr int stage_k(int f8) { return f8 ? 128 : 64; }

// The hardware square root (within 1 ulp of fp32), for the ReLU^2
// derivative 2 sqrt(a) whose product is rounded to bf16: sqrtf compiles to a
// correctly rounded sequence of about fifteen instructions per element.
__device__ __forceinline__ float sqrt_fast(float x) { return __builtin_amdgcn_sqrtf(x); }

// max of three finite floats in one instruction (fmaxf quiets NaN operands
// first, one more instruction per operand)
__device__ __forceinline__ float fmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// element idx = 16 j + e of a lane's accumulator row acc[0..TN)[0..16), by a
// select tree over the index bits (per-lane index, no dynamic register access)
template <int TN>
__device__ __forceinline__ float pick_acc(const f32x16_t (&row)[TN], int idx) {
  static_assert((TN & (TN - 1)) == 0 && TN <= 4, "TN: 1, 2 or 4");
  const int j = idx >> 4;
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float x = row[0][e];
#pragma unroll
    for (int jj = 1; jj < TN; ++jj) x = j == jj ? row[jj][e] : x;
    v[e] = x;
  }
#pragma unroll
  for (int h = 8; h >= 1; h >>= 1) {
    const bool hi = (idx & h) != 0;
#pragma unroll
    for (int k = 0; k < h; ++k) v[k] = hi ? v[k + h] : v[k];
  }
  return v[0];
}
// Workgroup shape per tile size: 256x256 tiles use 8 waves (two per SIMD, so
// one wave's LDS waits overlap the other's MFMAs), 128x128 tiles use 4.  The
// waves form a (NT/128) x 2 grid; each wave owns 64 rows and BN/2 columns.
// (Four 128x128 waves, one per SIMD, read a third less LDS per MFMA and leave
// registers for a deeper operand prefetch, but measured slower here: a lone
// wave per SIMD leaves every fragment-read and barrier latency exposed.)
template <int BM, int BN>
struct Cfg {
  static constexpr int NT = BM == 256 ? 512 : 256;
  static constexpr int WAVES_M = NT / 128;
  static constexpr int WM = BM / WAVES_M, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
};

// k-contiguous LDS tile: R rows of 64 k (128 B); 16-byte chunks XOR-swizzled
// by (r >> 1) & 7 so that 16 consecutive rows at one logical chunk (a
// fragment read by 16 lanes) hit 16 distinct bank groups (64 banks x 4 B).
__device__ __forceinline__ int lds_off_k(int r, int kc) { return r * 128 + ((kc ^ ((r >> 1) & 7)) << 4); }

// mn-contiguous LDS tile: 64 rows (k) of R elements (2R bytes) stored as in
// memory; 64-byte units XOR-swizzled by k & 3, so the 4 consecutive k rows of
// a transpose read land in 4 distinct bank groups.
template <int R>
__device__ __forceinline__ int lds_off_mn(int k, int i) {
  return k * (2 * R) + ((((i >> 5) ^ (k & 3))) << 6) + ((i & 31) << 1);
}

// mn-contiguous fp8 LDS tile: 128 rows (k) of R codes (R bytes) stored as in
// memory; 32-byte units XOR-swizzled by the row (R = 256: k & 7; R = 128:
// (k >> 1) & 3, two rows per 256-byte line of the 64 banks), so the 8
// consecutive k rows x 32 codes that half a wave's transpose read touches
// land in 8 distinct groups of 8 banks.
template <int R>
__device__ __forceinline__ int lds_off_mn8(int k, int m) {
  static_assert(R == 128 || R == 256, "fp8 mn tile rows of 128 or 256 codes");
  const int f = R == 256 ? (k & 7) : ((k >> 1) & 3);
  return k * R + (((m >> 5) ^ f) << 5) + (m & 31);
}

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;

// transpose read: within each 16-lane group, lane j receives element j % 4 of
// the 8 bytes loaded by lanes 4t + j / 4 (t = 0..3)
__device__ __forceinline__ v4s_t ds_read_tr(const char* lds_generic, int byte_off) {
  const __attribute__((address_space(3))) char* base =
      (const __attribute__((address_space(3))) char*)(lds_generic);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(base + byte_off));
}

// 8-bit transpose read: within each 16-lane group, lane j receives byte j % 8
// of the 8 bytes loaded by lanes 2t + j / 8 (t = 0..7), as its byte t
__device__ __forceinline__ v2i_t ds_read_tr8(const char* lds_generic, int byte_off) {
  const __attribute__((address_space(3))) char* base =
      (const __attribute__((address_space(3))) char*)(lds_generic);
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(base + byte_off));
}

// ---------------------------------------------------------------------------
// global -> register staging of one operand tile (R rows x 128 bytes of k):
// R*8 chunks of 16 B, R*8/NT per thread, for either layout.  ES = bytes per
// element (2: bf16, 1: fp8 codes).
// ---------------------------------------------------------------------------
template <int R, bool KC, int NT, int ES = 2>
struct TileLoader {
  static constexpr int kRegs = R * 8 / NT;
  static constexpr int EPC = 16 / ES;   // elements per 16-byte chunk
  static constexpr int KBK = 128 / ES;  // k elements per stage
  uint4 v[kRegs];

  template <bool GUARD>
  __device__ __forceinline__ void load(const void* __restrict__ Xv, long long ld, int row0, int rows,
                                       int k0, int K, int tid) {
    const char* __restrict__ Xb = reinterpret_cast<const char*>(Xv);
    const uint16_t* __restrict__ X = reinterpret_cast<const uint16_t*>(Xv);
    const bool full = !GUARD || ((row0 + R <= rows) && (k0 + KBK <= K));
#pragma unroll
    for (int i = 0; i < kRegs; ++i) {
      const int c = tid + NT * i;
      int gr, gk;
      if constexpr (KC) {
        gr = row0 + (c >> 3);
        gk = k0 + (c & 7) * EPC;
      } else {
        gk = k0 + c / (R / EPC);
        gr = row0 + (c % (R / EPC)) * EPC;
      }
      const long long base = KC ? (long long)gr * ld + gk : (long long)gk * ld + gr;
      if (full) {
        v[i] = *reinterpret_cast<const uint4*>(Xb + base * ES);
      } else if constexpr (ES == 1) {
        // fp8: K and an m/n-contiguous operand's rows are multiples of 16
        // (checked on the host), so a chunk is wholly inside or outside
        v[i] = (gr < rows && gk < K) ? *reinterpret_cast<const uint4*>(Xb + base) : make_uint4(0, 0, 0, 0);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t lo = 0, hi = 0;
          if constexpr (KC) {
            if (gr < rows && gk + 2 * j < K) lo = X[base + 2 * j];
            if (gr < rows && gk + 2 * j + 1 < K) hi = X[base + 2 * j + 1];
          } else {
            if (gk < K && gr + 2 * j < rows) lo = X[base + 2 * j];
            if (gk < K && gr + 2 * j + 1 < rows) hi = X[base + 2 * j + 1];
          }
          w[j] = lo | (hi << 16);
        }
        v[i] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  // Direct global -> LDS copy of a whole interior tile (global_load_lds_dwordx4):
  // lane l of wave w in round i fills the 16-byte LDS slot 256 i + 64 w + l of
  // the tile, so each lane fetches the global chunk that the swizzled layout
  // places in that slot.
  __device__ __forceinline__ static void load_direct(const void* __restrict__ Xv, long long ld, int row0,
                                                     int k0, char* lds, int tid) {
    const char* __restrict__ X = reinterpret_cast<const char*>(Xv);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int i = 0; i < kRegs; ++i) {
      const int slot = tid + NT * i;
      long long src;
      if constexpr (KC) {
        const int r = slot >> 3, kc = (slot & 7) ^ ((r >> 1) & 7);
        src = (long long)(row0 + r) * ld + k0 + kc * EPC;
      } else if constexpr (ES == 2) {
        const int b = slot * 16;
        const int k = b / (2 * R), rb = b % (2 * R);
        const int i_el = (((rb >> 6) ^ (k & 3)) << 5) + ((rb & 63) >> 1);
        src = (long long)(k0 + k) * ld + row0 + i_el;
      } else {
        src = (long long)(k0 + (slot * 16) / R) * ld + row0 + mn8_elem(slot);
      }
      __attribute__((address_space(3))) char* dst =
          (__attribute__((address_space(3))) char*)(lds) + (NT * i + 64 * wave) * 16;
      __builtin_amdgcn_global_load_lds((const void*)(X + src * ES), (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  }

  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kRegs; ++i) {
      const int c = tid + NT * i;
      const int off = KC ? lds_off_k(c >> 3, c & 7)
                         : (ES == 2 ? lds_off_mn<R>(c / (R / 8), (c % (R / 8)) * 8)
                                    : lds_off_mn8<R>(c / (R / 16), (c % (R / 16)) * 16));
      *reinterpret_cast<uint4*>(lds + off) = v[i];
    }
  }

  // MFMA fragment of rows r0 .. r0+31 (r0 a multiple of 32), k-step ks: lane
  // l holds row r0 + l % 32 and k = 16 ks + 8 (l / 32) + 0..7
  __device__ __forceinline__ static bf16x8_t frag(const char* lds, int r0, int ks, int lane) {
    if constexpr (KC) {
      return *reinterpret_cast<const bf16x8_t*>(lds + lds_off_k(r0 + (lane & 31), ks * 2 + (lane >> 5)));
    } else {
      const int g = lane >> 4, m = lane & 15;
      const int i = r0 + 16 * (g & 1) + 4 * (m & 3);
      const int k = ks * 16 + 8 * (g >> 1) + (m >> 2);
      const v4s_t a = ds_read_tr(lds, lds_off_mn<R>(k, i));
      const v4s_t b = ds_read_tr(lds, lds_off_mn<R>(k + 4, i));
      bf16x8_t f;
      f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
      f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
      return f;
    }
  }

  // fp8 fragment of rows r0 .. r0+31, k-step ks (64 codes): lane l holds row
  // r0 + l % 32 and the 32 codes of 16-byte chunks 4 ks + 2 (l / 32) + {0, 1}.
  // (Any assignment of the 64 k values to (lane half, byte) works as long as
  // both operands use the same one: the MFMA pairs equal positions.)
  // An m/n-contiguous tile gives the same assignment (byte p of lane half h
  // = k 64 ks + 32 h + p) through four transpose reads: read q of lane l
  // loads the 8 codes at k row 64 ks + 32 (l / 32) + 8 q + (l % 16) / 2,
  // columns r0 + 16 ((l / 16) % 2) + 8 (l % 2) + 0..7, so lane l receives
  // column r0 + l % 32 of k rows 64 ks + 32 (l / 32) + 8 q + 0..7.
  __device__ __forceinline__ static i32x8_t frag8(const char* lds, int r0, int ks, int lane) {
    i32x8_t f;
    if constexpr (KC) {
      // native vector loads (a struct-typed load here makes the compiler wait
      // for every direct global -> LDS load in flight before the read)
      typedef int i32x4_t __attribute__((ext_vector_type(4)));
      const int r = r0 + (lane & 31), c = ks * 4 + (lane >> 5) * 2;
      const i32x4_t a = *reinterpret_cast<const i32x4_t*>(lds + lds_off_k(r, c));
      const i32x4_t b = *reinterpret_cast<const i32x4_t*>(lds + lds_off_k(r, c + 1));
      f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
      f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    } else {
      const int m = r0 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
      const int kb = ks * 64 + 32 * (lane >> 5) + ((lane & 15) >> 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v2i_t x = ds_read_tr8(lds, lds_off_mn8<R>(kb + 8 * q, m));
        f[2 * q] = x[0];
        f[2 * q + 1] = x[1];
      }
    }
    return f;
  }

  // element offset (along the rows) of the 16-byte chunk that the swizzled
  // mn-contiguous fp8 layout places in LDS slot `slot` (k row slot * 16 / R)
  __device__ __forceinline__ static int mn8_elem(int slot) {
    const int b = slot * 16, k = b / R, rb = b % R;
    const int f = R == 256 ? (k & 7) : ((k >> 1) & 3);
    return (((rb >> 5) ^ f) << 5) + (rb & 31);
  }
};

// ---------------------------------------------------------------------------
// Output stores are non-temporal: a tile's outputs are written once and read
// by a later kernel, and marked so they do not displace the operand panels
// the other workgroups are streaming (the d20 MLP product with bf16 output:
// 0.79 -> 0.74 ms; 65536x1280x1280: 0.20 -> 0.185 ms).
// ---------------------------------------------------------------------------
// (st_nt: common.h)

// ---------------------------------------------------------------------------
// epilogues on 4 consecutive columns n .. n+3 of row m
// ---------------------------------------------------------------------------
template <int EPI>
__device__ __forceinline__ void epi4(const GemmArgs& p, int bi, int m, int n, const float* v, long long coff,
                                     float& amx, bool have_c = false, float4 cpre = make_float4(0.f, 0.f, 0.f, 0.f)) {
  const bool full = (n + 3 < p.N);
  if constexpr (EPI == EPI_F16) {
    _Float16* H = reinterpret_cast<_Float16*>(p.C) + (long long)bi * p.sC + (long long)m * p.ldc + n;
    for (int j = 0; j < 4; ++j)
      if (n + j < p.N) H[j] = (_Float16)v[j];
    return;
  }
  if constexpr (EPI == EPI_F32 || EPI == EPI_RESID) {
    float* C = reinterpret_cast<float*>(p.C) + (long long)bi * p.sC + coff + (long long)m * p.ldc + n;
    if (full) {
      float4 o = make_float4(v[0], v[1], v[2], v[3]);
      if (EPI == EPI_RESID || p.beta != 0.f) {
        const float4 c = have_c ? cpre : *reinterpret_cast<const float4*>(C);
        const float b = (EPI == EPI_RESID) ? 1.f : p.beta;
        o.x += b * c.x; o.y += b * c.y; o.z += b * c.z; o.w += b * c.w;
      }
      st_nt(C, o);
    } else {
      for (int j = 0; j < 4; ++j)
        if (n + j < p.N) {
          float o = v[j];
          if (EPI == EPI_RESID) o += C[j];
          else if (p.beta != 0.f) o += p.beta * C[j];
          C[j] = o;
        }
    }
  } else if constexpr (EPI == EPI_BF16 || EPI == EPI_RELU2 || EPI == EPI_DRELU2 || EPI == EPI_NS_POLY) {
    uint16_t* C = reinterpret_cast<uint16_t*>(p.C) + (long long)bi * p.sC + (long long)m * p.ldc + n;
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = v[j];
    if constexpr (EPI == EPI_RELU2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) { const float r = fmaxf(o[j], 0.f); o[j] = r * r; }
    }
    if constexpr (EPI == EPI_DRELU2) {
      const uint16_t* a = reinterpret_cast<const uint16_t*>(p.aux) + (long long)bi * p.sAux + (long long)m * p.ldaux + n;
      for (int j = 0; j < 4; ++j) o[j] = (n + j < p.N) ? o[j] * 2.f * sqrt_fast(bf2f(a[j])) : 0.f;
    }
    if constexpr (EPI == EPI_NS_POLY) {
      const uint16_t* a = reinterpret_cast<const uint16_t*>(p.aux) + (long long)bi * p.sAux + (long long)m * p.ldaux + n;
      for (int j = 0; j < 4; ++j) o[j] = (n + j < p.N) ? o[j] + p.beta * bf2f(a[j]) : 0.f;
    }
    if (full) {
      const uint2 w = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
      st_nt(C, w);
      if (p.amax)
        amx = fmaxf(amx, fmaxf(fmaxf(fabsf(lo_bf(w.x)), fabsf(hi_bf(w.x))), fmaxf(fabsf(lo_bf(w.y)), fabsf(hi_bf(w.y)))));
    } else {
      for (int j = 0; j < 4; ++j)
        if (n + j < p.N) {
          const uint16_t b = f2bf(o[j]);
          C[j] = b;
          if (p.amax) amx = fmaxf(amx, fabsf(bf2f(b)));
        }
    }

  }
}


// bf16-output epilogues on 8 consecutive columns n .. n+7 of row m (16-byte
// stores; C rows and the saved activation 16-byte aligned)
template <int EPI>
__device__ __forceinline__ void epi8(const GemmArgs& p, int bi, int m, int n, const float* v, float& amx,
                                     uint4 aux_w) {
  static_assert(EPI == EPI_BF16 || EPI == EPI_RELU2 || EPI == EPI_DRELU2 || EPI == EPI_NS_POLY || EPI == EPI_F16,
                "16-bit store epilogues");
  const bool full = (n + 7 < p.N);
  if constexpr (EPI == EPI_F16) {
    _Float16* H = reinterpret_cast<_Float16*>(p.C) + (long long)bi * p.sC + (long long)m * p.ldc + n;
    if (full) {
      typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
      h8_t h;
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = (_Float16)v[j];
      const uint4 hw = *reinterpret_cast<const uint4*>(&h);
      st_nt(H, hw);
    } else {
      for (int j = 0; j < 8; ++j)
        if (n + j < p.N) H[j] = (_Float16)v[j];
    }
    return;
  }
  uint16_t* C = reinterpret_cast<uint16_t*>(p.C) + (long long)bi * p.sC + (long long)m * p.ldc + n;
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = v[j];
  if constexpr (EPI == EPI_RELU2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) { const float r = fmaxf(o[j], 0.f); o[j] = r * r; }
  }
  if constexpr (EPI == EPI_DRELU2) {
    if (full) {
      const uint32_t w[4] = {aux_w.x, aux_w.y, aux_w.z, aux_w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] *= 2.f * sqrt_fast(lo_bf(w[j]));
        o[2 * j + 1] *= 2.f * sqrt_fast(hi_bf(w[j]));
      }
    } else {
      const uint16_t* a = reinterpret_cast<const uint16_t*>(p.aux) + (long long)bi * p.sAux + (long long)m * p.ldaux + n;
      for (int j = 0; j < 8; ++j) o[j] = (n + j < p.N) ? o[j] * 2.f * sqrt_fast(bf2f(a[j])) : 0.f;
    }
  }
  if constexpr (EPI == EPI_NS_POLY) {
    if (full) {
      const uint32_t w[4] = {aux_w.x, aux_w.y, aux_w.z, aux_w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] += p.beta * lo_bf(w[j]);
        o[2 * j + 1] += p.beta * hi_bf(w[j]);
      }
    } else {
      const uint16_t* a = reinterpret_cast<const uint16_t*>(p.aux) + (long long)bi * p.sAux + (long long)m * p.ldaux + n;
      for (int j = 0; j < 8; ++j) o[j] = (n + j < p.N) ? o[j] + p.beta * bf2f(a[j]) : 0.f;
    }
  }
  if (full) {
    const uint4 w = make_uint4(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]), pack_bf2(o[4], o[5]), pack_bf2(o[6], o[7]));
    st_nt(C, w);
    if (p.amax) {
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) amx = fmaxf(amx, fmaxf(fabsf(lo_bf(ww[j])), fabsf(hi_bf(ww[j]))));
    }
  } else {
    for (int j = 0; j < 8; ++j)
      if (n + j < p.N) {
        const uint16_t b = f2bf(o[j]);
        C[j] = b;
        if (p.amax) amx = fmaxf(amx, fabsf(bf2f(b)));
      }
  }
}

// 16-bit outputs already converted (8 consecutive columns n .. n+7 of row m
// as one 16-byte word): store, and the amax of the stored values
template <int EPI>
__device__ __forceinline__ void st16(const GemmArgs& p, int bi, int m, int n, uint4 w, float& amx) {
  uint16_t* C = reinterpret_cast<uint16_t*>(p.C) + (long long)bi * p.sC + (long long)m * p.ldc + n;
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  if (n + 7 < p.N) {
    st_nt(C, w);
    if (EPI != EPI_F16 && p.amax) {
#pragma unroll
      for (int j = 0; j < 4; ++j) amx = fmaxf(amx, fmaxf(fabsf(lo_bf(ww[j])), fabsf(hi_bf(ww[j]))));
    }
  } else {
    for (int j = 0; j < 8; ++j)
      if (n + j < p.N) {
        const uint16_t b = (uint16_t)(ww[j >> 1] >> (16 * (j & 1)));
        C[j] = b;
        if (EPI != EPI_F16 && p.amax) amx = fmaxf(amx, fabsf(bf2f(b)));
      }
  }
}

// ---------------------------------------------------------------------------
// K loop: double-buffered LDS stages, fragments double-buffered in registers,
// and (for interior tiles, GUARD = false) an explicit interleave of MFMAs with
// the global loads, LDS fragment reads and LDS stores of the same iteration.
// ---------------------------------------------------------------------------
template <int BM, int BN, bool AK, bool BKC, bool GUARD, int F8>
__device__ __forceinline__ void mainloop(const GemmArgs& p, const void* A, const void* B, int m0, int n0,
                                         int kt0, int nk, char* smem, int tid,
                                         f32x16_t (&acc)[Cfg<BM, BN>::TM][Cfg<BM, BN>::TN]) {
  constexpr int NT = Cfg<BM, BN>::NT;
  constexpr int WM = Cfg<BM, BN>::WM, WN = Cfg<BM, BN>::WN, TM = Cfg<BM, BN>::TM, TN = Cfg<BM, BN>::TN;
  constexpr int ES = F8 ? 1 : 2;
  constexpr int KBK = stage_k(F8);
  using LA = TileLoader<BM, AK, NT, ES>;
  using LB = TileLoader<BN, BKC, NT, ES>;
  using FragT = typename std::conditional<F8 != 0, i32x8_t, bf16x8_t>::type;
  constexpr int A_BYTES = BM * 128, STAGE = (BM + BN) * 128;
  constexpr int KS = F8 ? 2 : 4;                                 // MFMA k-steps per stage
  constexpr int NM = TM * TN;                                    // MFMAs per k-step
  constexpr int NV = LA::kRegs + LB::kRegs;                      // global loads per tile
  constexpr int ND = F8 ? (AK ? 2 : 4) * TM + (BKC ? 2 : 4) * TN : (AK ? 1 : 2) * TM + (BKC ? 1 : 2) * TN;  // LDS reads per k-step
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  if (nk <= 0) return;

  auto frag_a = [&](const char* base, int r0, int ks) -> FragT {
    if constexpr (F8) return LA::frag8(base, r0, ks, lane);
    else return LA::frag(base, r0, ks, lane);
  };
  auto frag_b = [&](const char* base, int r0, int ks) -> FragT {
    if constexpr (F8) return LB::frag8(base, r0, ks, lane);
    else return LB::frag(base, r0, ks, lane);
  };

  LA la;
  LB lb;
  if constexpr (GUARD) {
    la.template load<true>(A, p.lda, m0, p.M, kt0 * KBK, p.K, tid);
    lb.template load<true>(B, p.ldb, n0, p.N, kt0 * KBK, p.K, tid);
    la.store(smem, tid);
    lb.store(smem + A_BYTES, tid);
  } else {
    LA::load_direct(A, p.lda, m0, kt0 * KBK, smem, tid);
    LB::load_direct(B, p.ldb, n0, kt0 * KBK, smem + A_BYTES, tid);
  }
  __syncthreads();

  FragT fa[2][TM], fb[2][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) fa[0][i] = frag_a(smem, wm * WM + i * 32, 0);
#pragma unroll
  for (int j = 0; j < TN; ++j) fb[0][j] = frag_b(smem + A_BYTES, wn * WN + j * 32, 0);

  for (int kt = 0; kt < nk; ++kt) {
    const char* sa = smem + (kt & 1) * STAGE;
    const char* sb = sa + A_BYTES;
    char* so = smem + ((kt + 1) & 1) * STAGE;
    // next tile (the last iteration reloads its own tile: harmless, no branch)
    const int kn = (kt0 + (kt + 1 < nk ? kt + 1 : kt)) * KBK;
    if constexpr (GUARD) {
      la.template load<true>(A, p.lda, m0, p.M, kn, p.K, tid);
      lb.template load<true>(B, p.ldb, n0, p.N, kn, p.K, tid);
    } else {
      // the other stage was last read before the previous barrier
      LA::load_direct(A, p.lda, m0, kn, so, tid);
      LB::load_direct(B, p.ldb, n0, kn, so + A_BYTES, tid);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (ks + 1 < KS) {
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[nxt][i] = frag_a(sa, wm * WM + i * 32, ks + 1);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[nxt][j] = frag_b(sb, wn * WN + j * 32, ks + 1);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (F8)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb[cur][j], fa[cur][i], acc[i][j], f8_fmt_b(F8), f8_fmt_a(F8), 0, 127, 0, 127);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cur][j], fa[cur][i], acc[i][j], 0, 0, 0);
        }
      if constexpr (GUARD) {
        if (ks + 1 == KS) {
          la.store(so, tid);
          lb.store(so + A_BYTES, tid);
        }
      }
    }
    if constexpr (!GUARD) {
      // k-step 0: MFMAs with the direct loads and the fragment reads of k-step 1;
      // later k-steps: MFMAs with the next fragment reads
#pragma unroll
      for (int x = 0; x < NM; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (x < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        if (x < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int ks = 1; ks < KS; ++ks)
#pragma unroll
        for (int x = 0; x < NM; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (ks + 1 < KS && x < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[0][i] = frag_a(so, wm * WM + i * 32, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = frag_b(so + A_BYTES, wn * WN + j * 32, 0);
  }
}

// ---------------------------------------------------------------------------
// Interior tiles: two LDS blocks of 128 bytes of k per operand row (64 bf16
// or 128 fp8 codes; the layouts of the general loop), double buffered, loaded
// by direct buffer -> LDS loads issued as instructions the compiler does not
// model (with the builtin it makes every LDS read wait for all loads in
// flight); the loop carries its own waits.  Whole 128-byte rows per block
// matter: a wave's 16-byte-per-lane load then covers whole cache lines, while
// 64-byte half rows fetch each line from L2 twice and stall the address unit
// on the L1.  Per-lane byte offsets are loop invariant; the k position goes
// in the scalar offset.
// ---------------------------------------------------------------------------
typedef int v4i_t __attribute__((ext_vector_type(4)));

// buffer resource (raw bytes, range num_bytes) from wave-uniform values
__device__ __forceinline__ v4i_t dma_rsrc(const void* base, long long num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int)min(num_bytes, (long long)0x7fffffff));
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from rsrc at voff + soff into LDS at lds + 16 lane (lds
// wave-uniform).  No register results; "memory" keeps LDS accesses in place;
// M0 is set here only and nothing compiled in the GEMM kernel reads it.
__device__ __forceinline__ void dma16(v4i_t rsrc, int voff, int soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %0, %2 offen lds"
               :: "s"(rsrc), "v"(voff), "s"(soff), "s"(lds) : "memory");
}

// True when every byte offset of the block loads fits 31 bits.
__device__ __forceinline__ bool dma_fits(const GemmArgs& p, int BM, int BN, bool AK, bool BKC, int ES) {
  const long long ea = AK ? (long long)BM * p.lda * ES : (long long)p.K * p.lda * ES;
  const long long eb = BKC ? (long long)BN * p.ldb * ES : (long long)p.K * p.ldb * ES;
  return ea < 0x7fffffffLL && eb < 0x7fffffffLL;
}

// The loads of one operand tile (R rows x 128 bytes of k) into the LDS
// layout TileLoader reads fragments from: lane l of wave w in round i fills
// the 16-byte slot NT i + 64 w + l.
template <int R, bool KC, int NT, int ES>
struct DmaOperand {
  static constexpr int NL = R * 8 / NT;  // 16-byte loads per thread per block
  v4i_t rsrc;
  int voff[NL];
  long long kstep;  // bytes per k element along the loaded direction

  // nrows: rows (KC) or elements (MN, a multiple of 16 / ES) of the operand from
  // row0 on; a tile reaching past them re-reads the last valid row / 16-byte
  // chunk instead (its products land in output rows / columns that are never
  // stored), so every load stays inside the operand
  __device__ __forceinline__ void init(const char* X, long long ld, int row0, int nrows, int K, int tid) {
    if constexpr (KC) {
      rsrc = dma_rsrc(X + (long long)row0 * ld * ES, (long long)min(R, nrows) * ld * ES);
      kstep = ES;
    } else {
      rsrc = dma_rsrc(X + (long long)row0 * ES, ((long long)K * ld - row0) * ES);
      kstep = ld * ES;
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int slot = tid + NT * i;
      if constexpr (KC) {
        const int r = min(slot >> 3, nrows - 1), kc = (slot & 7) ^ (((slot >> 3) >> 1) & 7);
        voff[i] = (int)(((long long)r * ld + kc * (16 / ES)) * ES);
      } else if constexpr (ES == 2) {
        const int b = slot * 16;
        const int k = b / (2 * R), rb = b % (2 * R);
        const int i_el = min((((rb >> 6) ^ (k & 3)) << 5) + ((rb & 63) >> 1), nrows - 8);
        voff[i] = (int)(((long long)k * ld + i_el) * 2);
      } else {
        const int k = (slot * 16) / R;
        const int i_el = min(TileLoader<R, false, NT, 1>::mn8_elem(slot), nrows - 16);
        voff[i] = (int)((long long)k * ld + i_el);
      }
    }
  }
};

// Block kt of the loop: barrier (block kt landed, every wave done reading
// block kt - 1), then walk the block's k-steps with the fragments of each
// k-step read while the MFMAs of the previous one run; the last k-step's
// MFMAs run after the next barrier, covering the first fragment reads of the
// next block.  The loads of block kt + 1 (into the other buffer) are spread
// over the first DMA_PHASES k-steps, between the two halves of an MFMA batch
// (slightly faster than one burst after the barrier, which backs up the
// address unit; spreading them further leaves the last ones too little time).
constexpr int DMA_PHASES = 2;
template <int BM, int BN, bool AK, bool BKC, int F8>
__device__ __forceinline__ void mainloop_dma(const GemmArgs& p, const char* A, const char* B, int m0, int n0,
                                             int kt0, int nk, char* smem, int tid,
                                             f32x16_t (&acc)[Cfg<BM, BN>::TM][Cfg<BM, BN>::TN]) {
  constexpr int NT = Cfg<BM, BN>::NT;
  constexpr int WM = Cfg<BM, BN>::WM, WN = Cfg<BM, BN>::WN, TM = Cfg<BM, BN>::TM, TN = Cfg<BM, BN>::TN;
  constexpr int ES = F8 ? 1 : 2;
  constexpr int KBK = stage_k(F8);                // k elements per block
  constexpr int KS = F8 ? 2 : 4;                  // MFMA k-steps per block
  constexpr int A_BYTES = BM * 128, STAGE = (BM + BN) * 128;
  using OA = DmaOperand<BM, AK, NT, ES>;
  using OB = DmaOperand<BN, BKC, NT, ES>;
  using LA = TileLoader<BM, AK, NT, ES>;
  using LB = TileLoader<BN, BKC, NT, ES>;
  using FragT = typename std::conditional<F8 != 0, i32x8_t, bf16x8_t>::type;
  constexpr int NV = OA::NL + OB::NL;                                   // loads per thread per block
  constexpr int PH = DMA_PHASES < KS ? DMA_PHASES : KS;                 // k-steps the loads spread over
  constexpr int PER = (NV + PH - 1) / PH;                               // loads per k-step
  static_assert(KS % 2 == 0, "fragment buffers alternate within a block");
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  if (nk <= 0) return;
  OA oa;
  OB ob;
  oa.init(A, p.lda, m0, p.M - m0, p.K, tid);
  ob.init(B, p.ldb, n0, p.N - n0, p.K, tid);
  // loads [PER ph, PER (ph + 1)) of block kt (clamped: the trailing re-load
  // lands in a buffer never read again)
  auto issue = [&](int kt, int ph) {
    const int k0 = (kt0 + min(kt, nk - 1)) * KBK;
    char* so = smem + (kt & 1) * STAGE;
    const int soa = __builtin_amdgcn_readfirstlane((int)(k0 * oa.kstep));
    const int sob = __builtin_amdgcn_readfirstlane((int)(k0 * ob.kstep));
#pragma unroll
    for (int d = 0; d < NV; ++d) {
      if (d / PER != ph) continue;
      if (d < OA::NL)
        dma16(oa.rsrc, oa.voff[d], soa,
              (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(so + (NT * d + 64 * wave) * 16));
      else
        dma16(ob.rsrc, ob.voff[d - OA::NL], sob,
              (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(so + A_BYTES +
                                                                          (NT * (d - OA::NL) + 64 * wave) * 16));
    }
  };
  auto issue_all = [&](int kt) {
#pragma unroll
    for (int ph = 0; ph < PH; ++ph) issue(kt, ph);
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): block landed, this wave's reads done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  FragT f0a[TM], f0b[TN], f1a[TM], f1b[TN];
  auto read = [&](const char* st, int ks, FragT (&fa)[TM], FragT (&fb)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (F8) fa[i] = LA::frag8(st, wm * WM + i * 32, ks, lane);
      else fa[i] = LA::frag(st, wm * WM + i * 32, ks, lane);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (F8) fb[j] = LB::frag8(st + A_BYTES, wn * WN + j * 32, ks, lane);
      else fb[j] = LB::frag(st + A_BYTES, wn * WN + j * 32, ks, lane);
    }
  };
  // one MFMA batch (a k-step) with the loads of phase ph of block kt between
  // its halves (ph < 0: none)
  auto mfma = [&](const FragT (&fa)[TM], const FragT (&fb)[TN], int kt, int ph) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i == TM / 2 && ph >= 0 && ph < PH) {
        __builtin_amdgcn_sched_barrier(0);
        issue(kt, ph);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (F8)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], f8_fmt_b(F8),
                                                                      f8_fmt_a(F8), 0, 127, 0, 127);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
      }
    }
  };
  // k-steps 1 .. KS-1 of block st: read k-step ks while the MFMAs of ks - 1
  // run (scheduling fences keep each read batch ahead of the MFMA batch that
  // covers it; left alone, the scheduler sinks reads next to their uses)
  auto body = [&](const char* st, int kt) {
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) {
      if (ks & 1) read(st, ks, f1a, f1b);
      else read(st, ks, f0a, f0b);
      __builtin_amdgcn_sched_barrier(0);
      if (ks & 1) mfma(f0a, f0b, kt + 1, ks);
      else mfma(f1a, f1b, kt + 1, ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  issue_all(0);
  barrier();
  read(smem, 0, f0a, f0b);
  issue(1, 0);
  body(smem, 0);
  for (int kt = 1; kt < nk; ++kt) {
    const char* st = smem + (kt & 1) * STAGE;
    barrier();
    read(st, 0, f0a, f0b);
    __builtin_amdgcn_sched_barrier(0);
    mfma(f1a, f1b, kt + 1, 0);  // last k-step of block kt - 1
    __builtin_amdgcn_sched_barrier(0);
    body(st, kt);
  }
  mfma(f1a, f1b, 0, -1);
  // drain the trailing loads before the LDS is reused by the epilogue
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF70);
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int BM, int BN, bool AK, bool BKC, int EPI, int F8>
__global__ void __launch_bounds__((Cfg<BM, BN>::NT), 1) gemm_kernel(GemmArgs p) {
  constexpr int WM = Cfg<BM, BN>::WM, WN = Cfg<BM, BN>::WN, TM = Cfg<BM, BN>::TM, TN = Cfg<BM, BN>::TN;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  // The dispatcher hands workgroup x + gx y to XCD (x + gx y) % 8; remapping
  // that linear id gives each XCD a contiguous run of (batch/split, tile)
  // order, so the blocks resident on one XCD share a k range and neighbouring
  // row and column panels in its L2.
  const int nblk = gridDim.x * gridDim.y;
  const int lin = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, nblk);
  const int yb = lin / gridDim.x;
  const int lid = lin - yb * gridDim.x;
  int tile_m, tile_n;
  if (p.sym) {
    // upper triangle of a square tile grid, row by row (row r holds tiles_n - r tiles)
    int r = 0, rem = lid;
    while (rem >= tiles_n - r) rem -= tiles_n - r++;
    tile_m = r;
    tile_n = r + rem;
  } else {
    constexpr int GM = 4;
    const int group = lid / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsz = min(tiles_m - first_m, GM);
    const int in_group = lid - group * GM * tiles_n;
    tile_m = first_m + in_group % gsz;
    tile_n = in_group / gsz;
  }
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  const int bi = yb / p.k_split, split = yb % p.k_split;
  constexpr int KBK = stage_k(F8);
  const int nk_all = (p.K + KBK - 1) / KBK;
  const int nk_per = (nk_all + p.k_split - 1) / p.k_split;
  const int kt0 = split * nk_per;
  const int nk = max(0, min(nk_all, kt0 + nk_per) - kt0);

  constexpr int ES = F8 ? 1 : 2;
  const char* A = reinterpret_cast<const char*>(p.A) + (long long)bi * p.sA * ES;
  const char* B = reinterpret_cast<const char*>(p.B) + (long long)bi * p.sB * ES;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // the block-load loop takes every tile whose K is whole blocks; a tile
  // reaching past M or N needs that dimension a multiple of 8 bf16 / 16 fp8
  // elements when it is the contiguous one (16-byte chunks either wholly
  // inside or outside)
  const bool fast = (p.K % KBK == 0) && (m0 + BM <= p.M || AK || p.M % (16 / ES) == 0) &&
                    (n0 + BN <= p.N || BKC || p.N % (16 / ES) == 0);
  const bool interior = (m0 + BM <= p.M) && (n0 + BN <= p.N) && (p.K % KBK == 0);
  if (fast && dma_fits(p, BM, BN, AK, BKC, ES))
    mainloop_dma<BM, BN, AK, BKC, F8>(p, A, B, m0, n0, kt0, nk, smem, tid, acc);
  else if (interior)
    mainloop<BM, BN, AK, BKC, false, F8>(p, A, B, m0, n0, kt0, nk, smem, tid, acc);
  else
    mainloop<BM, BN, AK, BKC, true, F8>(p, A, B, m0, n0, kt0, nk, smem, tid, acc);
  const int lr = lane & 31, lh = lane >> 5;
  if constexpr (F8 != 0) {
    // dequantise: the codes carry x * s_x, so the product carries s_a * s_b
    const float inv = 1.0f / (p.scale_a[0] * p.scale_b[0]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= inv;
  }

  // ----------------------------- epilogue ---------------------------------
  // Rotary embedding + RMS normalisation of q / k heads, applied to row block
  // i of the accumulators just before it is staged (one row block at a time
  // keeps the working set in registers).  Each wave owns 128 columns = one
  // head (tiles are 256 wide).  Lane row m holds head features
  // e = j*32 + 8g + 4lh + r; the rotation partner e + 64 sits in the same
  // lane at j + 2, the other half of the head in lane ^ 32.
  auto qkv_rows = [&](int i) {
    if constexpr (EPI == EPI_QKV) {
      static_assert(WN == 128, "EPI_QKV needs 128 columns per wave");
      const int nb = n0 + wn * WN;  // first column of this wave's head
      const int dmodel = p.n_head * 128;
      const int nkv = p.n_kv_head ? p.n_kv_head : p.n_head;
      if (nb >= dmodel + nkv * 128) return;  // v head (wave-uniform)
      const int m = m0 + wm * WM + i * 32 + lr;
      const int t = (m < p.M) ? m % p.row_T : 0;
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int e = j * 32 + 8 * g + 4 * lh;
          const float4 c4 = *reinterpret_cast<const float4*>(p.rope + (long long)t * 64 + e);
          const float4 s4 = *reinterpret_cast<const float4*>(p.rope + (long long)p.row_T * 64 + (long long)t * 64 + e);
          const float cc[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x1 = acc[i][j][4 * g + r], x2 = acc[i][j + 2][4 * g + r];
            const float y1 = x1 * cc[r] - x2 * sn[r], y2 = x1 * sn[r] + x2 * cc[r];
            acc[i][j][4 * g + r] = y1;
            acc[i][j + 2][4 * g + r] = y2;
            ss += y1 * y1 + y2 * y2;
          }
        }
      ss += __shfl_xor(ss, 32, 64);
      const float rr = 1.0f / sqrtf(ss / 128.f + 1e-6f);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= rr;
      if (lh == 0 && m < p.M) {
        if (nb < dmodel) p.part[(long long)m * p.n_head + nb / 128] = rr;
        else p.zt[(long long)m * nkv + (nb - dmodel) / 128] = rr;
      }
    }
  };
  if constexpr (EPI == EPI_CE_FWD) {
    // Per row: max and sum of exp over this wave's WN columns, merged with
    // the partner lane (lane ^ 32) that holds the other half of the columns.
    // Element (j, e) of a lane is column cb + 4 lh + 32 j + 8 (e >> 2) + (e & 3).
    const int cb = n0 + wn * WN;
    const bool fulln = cb + WN <= p.N;  // wave-uniform: every column of the wave exists
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm * WM + i * 32 + lr;
      int tgt = -1;
      if (m < p.M) {
        const int row_b = m / p.row_T, row_t = m - row_b * p.row_T;
        tgt = p.row_i[(long long)row_b * (p.row_T + 1) + row_t + 1] - p.col_offset;
      }
      if (fulln) {
        // No column checks.  The max is taken on the raw accumulators
        // (alpha > 0) with three-operand maxes (finite values: no NaN
        // quieting), the exponentials as exp2 with alpha log2(e) folded in,
        // and the target logit is picked by a select tree over its element
        // index instead of a compare and a store per element.
        float mr = acc[i][0][0];
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = (j == 0 ? 1 : 0); e < 16; e += 2)
            mr = (e + 1 < 16) ? fmax3(mr, acc[i][j][e], acc[i][j][e + 1]) : fmaxf(mr, acc[i][j][e]);
        mr = fmaxf(mr, __shfl_xor(mr, 32, 64));
        const int rel = tgt - cb - 4 * lh;  // 32 j + 8 g + u when this lane holds the target
        if (m < p.M && rel >= 0 && rel < WN && (rel & 4) == 0)
          p.zt[m] = pick_acc<TN>(acc[i], ((rel >> 5) << 4) | ((rel >> 1) & 12) | (rel & 3)) * p.alpha;
        const float a2 = p.alpha * 1.4426950408889634f, ms = mr * a2;
        float s = 0.f;
        const bool keep = p.C != nullptr;  // launch-uniform: the exponentials are stored
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i][j][e], a2, -ms));
            s += pe;
            if (keep) acc[i][j][e] = pe;
          }
        s += __shfl_xor(s, 32, 64);
        if (lh == 0 && m < p.M) reinterpret_cast<float2*>(p.part)[(long long)m * p.nparts + tile_n * 2 + wn] =
            make_float2(mr * p.alpha, s);
        continue;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int n = n0 + wn * WN + j * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
          const float z = acc[i][j][e] * p.alpha;
          if (n < p.N) mx = fmaxf(mx, z);
          if (n == tgt) p.zt[m] = z;
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float s = 0.f;
      const bool keep = p.C != nullptr;  // launch-uniform: the exponentials are stored
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int n = n0 + wn * WN + j * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
          const float pe = n < p.N ? __expf(acc[i][j][e] * p.alpha - mx) : 0.f;
          s += pe;
          if (keep) acc[i][j][e] = pe;
        }
      s += __shfl_xor(s, 32, 64);
      if (lh == 0 && m < p.M && n0 + wn * WN < p.N) {
        reinterpret_cast<float2*>(p.part)[(long long)m * p.nparts + tile_n * 2 + wn] = make_float2(mx, s);
      }
    }
  }
  // The staged store (for the cross-entropy forward: the exponentials exp(z - mx) as
  // fp16, when C is given; acc holds them already, so the scale is 1)
  constexpr int SE = EPI == EPI_CE_FWD ? (int)EPI_F16 : EPI;
  const float alpha_st = EPI == EPI_CE_FWD ? 1.f : p.alpha;
  if (EPI != EPI_CE_FWD || p.C != nullptr) {  // launch-uniform
    // split-K partials: split s writes its own slice of C (reduced afterwards)
    const long long coff = (SE == EPI_F32 && p.k_split > 1) ? (long long)split * p.split_stride : 0;
    // Coalesced epilogue: each wave stages its accumulators, 32 rows at a
    // time, in its own LDS region (16-byte chunks XOR-swizzled by row, so
    // both the row-per-lane writes and the row-contiguous reads are
    // conflict free), then applies the epilogue on 4-column chunks laid out
    // along rows: consecutive lanes touch consecutive 16-byte pieces of a row.
    constexpr int ROWB = WN * 4;                 // bytes per staged row
    constexpr int CH = WN / 4;                   // 16-byte chunks per row
    static_assert(32 * ROWB * (Cfg<BM, BN>::NT / 64) <= 2 * STAGE, "epilogue staging exceeds LDS");
    char* wbuf = smem + wave * 32 * ROWB;
    // DRELU2 reads the saved activation, NS_POLY the bf16 Gram matrix, at
    // every output: each 32-row block's words are fetched in one burst, the
    // first block's before the staging barrier, so their latency overlaps the
    // staging instead of being paid every few outputs
    constexpr int NIT = 32 * CH / 64;
    // bf16 stores go out 8 columns (16 bytes) per lane when rows are 16-byte
    // aligned: half the store instructions of the 4-column path
    constexpr bool W8E = SE == EPI_BF16 || SE == EPI_RELU2 || SE == EPI_DRELU2 || SE == EPI_QKV || SE == EPI_F16 ||
                         SE == EPI_NS_POLY;
    constexpr bool AUX8 = SE == EPI_DRELU2 || SE == EPI_NS_POLY;  // bf16 aux read per output
    constexpr int CH2 = CH / 2, NIT8 = 32 * CH2 / 64;
    // 16-bit outputs staged as such (below)
    constexpr bool PRE16 = SE == EPI_BF16 || SE == EPI_RELU2 || SE == EPI_QKV || SE == EPI_F16;
    constexpr int ROWB16 = WN * 2;
    const bool w8 = W8E && (p.ldc % 8 == 0) && (!AUX8 || p.ldaux % 8 == 0);
    // (the ReLU^2-derivative epilogue always takes the 8-column path: its
    // launches keep C and the saved activation 16-byte aligned, and the 4-column
    // path reads the activation per element)
    uint4 auxw8[AUX8 ? TM : 1][NIT8];
    auto fetch_aux = [&](int i) {
      if constexpr (AUX8) {
        const uint16_t* ab = reinterpret_cast<const uint16_t*>(p.aux) + (long long)bi * p.sAux;
#pragma unroll
        for (int it = 0; it < NIT8; ++it) {
          const int q = it * 64 + lane;
          const int m = m0 + wm * WM + i * 32 + q / CH2;
          const int n = n0 + wn * WN + (q % CH2) * 8;
          auxw8[i][it] = (w8 && m < p.M && n + 7 < p.N) ? *reinterpret_cast<const uint4*>(ab + (long long)m * p.ldaux + n)
                                                      : make_uint4(0, 0, 0, 0);
        }
      }
    };
    // Epilogues that read fp32 C per output (the residual add, the NS update
    // and fp32 with beta) fetch a row block's values in one burst before
    // staging it: read one at a time between the stores, each load would wait
    // out the stores before it (the compiler cannot tell the addresses apart)
    constexpr bool READS_C = SE == EPI_RESID || SE == EPI_F32;
    const bool cread = READS_C && (SE != EPI_F32 || p.beta != 0.f);
    float4 cpre[READS_C ? NIT : 1];
    auto fetch_c = [&](int i) {
      if constexpr (READS_C) {
        if (!cread) return;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int q = it * 64 + lane;
          const int m = m0 + wm * WM + i * 32 + q / CH;
          const int n = n0 + wn * WN + (q % CH) * 4;
          float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
          const float* Cb = reinterpret_cast<const float*>(p.C) + (long long)bi * p.sC + coff;
          if (m < p.M && n + 3 < p.N) x = *reinterpret_cast<const float4*>(Cb + (long long)m * p.ldc + n);
          cpre[it] = x;
        }
      }
    };
    // every row block's aux words at once (16 bytes per lane per 8 columns):
    // fetched between the stores of an earlier block, a load waits for those
    // stores to complete
#pragma unroll
    for (int i = 0; i < TM; ++i) fetch_aux(i);
    fetch_c(0);
    __syncthreads();  // every wave is done with the operand tiles
    float amx = 0.f;  // max |stored value| of this lane (bf16 epilogues with p.amax)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i > 0) {
        fetch_c(i);
      }
      qkv_rows(i);
      if (PRE16 && w8) {
        if constexpr (PRE16) {
          // Outputs whose epilogue is elementwise on the accumulator are
          // converted before staging: 16-bit rows of 2 WN bytes (16-byte
          // chunks of 8 columns XOR-swizzled by row), half the LDS bytes of
          // fp32 staging, and each lane reads back a finished 16-byte store.
          // Same arithmetic as the fp32-staged path (scale, ReLU^2, one
          // rounding), so the same bits.
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              float o[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                o[r] = acc[i][j][4 * g + r] * alpha_st;
                if constexpr (SE == EPI_RELU2) {
                  const float t = fmaxf(o[r], 0.f);
                  o[r] = t * t;
                }
              }
              uint2 w;
              if constexpr (SE == EPI_F16) {
                typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
                const h4_t h = {(_Float16)o[0], (_Float16)o[1], (_Float16)o[2], (_Float16)o[3]};
                w = __builtin_bit_cast(uint2, h);
              } else {
                w = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
              }
              const int c8 = (j * 32 + 8 * g) >> 3;
              *reinterpret_cast<uint2*>(wbuf + lr * ROWB16 + ((c8 ^ (lr & (CH2 - 1))) << 4) + 8 * lh) = w;
            }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
          for (int it = 0; it < NIT8; ++it) {
            const int q = it * 64 + lane;
            const int rr = q / CH2, cc = q % CH2;
            const uint4 w = *reinterpret_cast<const uint4*>(wbuf + rr * ROWB16 + ((cc ^ (rr & (CH2 - 1))) << 4));
            const int m = m0 + wm * WM + i * 32 + rr;
            const int n = n0 + wn * WN + cc * 8;
            if (m < p.M && n < p.N) st16<SE>(p, bi, m, n, w, amx);
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        continue;
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int cc = (j * 32 + 8 * g + 4 * lh) >> 2;
          *reinterpret_cast<float4*>(wbuf + lr * ROWB + ((cc ^ (lr & 15)) << 4)) =
              make_float4(acc[i][j][4 * g] * alpha_st, acc[i][j][4 * g + 1] * alpha_st,
                          acc[i][j][4 * g + 2] * alpha_st, acc[i][j][4 * g + 3] * alpha_st);
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (w8) {
        if constexpr (W8E) {
#pragma unroll
          for (int it = 0; it < NIT8; ++it) {
            const int q = it * 64 + lane;
            const int rr = q / CH2, cc = 2 * (q % CH2);
            const float4 a4 = *reinterpret_cast<const float4*>(wbuf + rr * ROWB + ((cc ^ (rr & 15)) << 4));
            const float4 b4 = *reinterpret_cast<const float4*>(wbuf + rr * ROWB + (((cc + 1) ^ (rr & 15)) << 4));
            const int m = m0 + wm * WM + i * 32 + rr;
            const int n = n0 + wn * WN + cc * 4;
            if (m < p.M && n < p.N) {
              const float v[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
              epi8<(SE == EPI_QKV ? (int)EPI_BF16 : SE)>(p, bi, m, n, v, amx, auxw8[AUX8 ? i : 0][it]);
            }
          }
        }
      } else {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int q = it * 64 + lane;
          const int rr = q / CH, cc = q % CH;
          const float4 v4 = *reinterpret_cast<const float4*>(wbuf + rr * ROWB + ((cc ^ (rr & 15)) << 4));
          const int m = m0 + wm * WM + i * 32 + rr;
          const int n = n0 + wn * WN + cc * 4;
          if (m < p.M && n < p.N) {
            const float v[4] = {v4.x, v4.y, v4.z, v4.w};
            if constexpr (READS_C)
              epi4<SE>(p, bi, m, n, v, coff, amx, cread && n + 3 < p.N, cpre[it]);
            else
              epi4<(SE == EPI_QKV ? (int)EPI_BF16 : SE)>(p, bi, m, n, v, coff, amx);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if constexpr (SE == EPI_BF16 || SE == EPI_RELU2 || SE == EPI_DRELU2) {
      if (p.amax) {  // launch-uniform
        const float wm_ = wave_max(amx);
        if (lane == 0)
          p.amax[((long long)blockIdx.x + (long long)gridDim.x * blockIdx.y) * (Cfg<BM, BN>::NT / 64) + wave] = wm_;
      }
    }
  }
}

template <int BM, int BN, bool AK, bool BKC, int EPI, int F8 = 0>
int launch_t(const GemmArgs& a, hipStream_t s) {
  const int tm = (a.M + BM - 1) / BM;
  const int tiles = a.sym ? tm * (tm + 1) / 2 : tm * ((a.N + BN - 1) / BN);
  dim3 grid(tiles, a.batch * a.k_split);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BKC, EPI, F8>), grid, dim3(Cfg<BM, BN>::NT), 0, s, a);
  GS_LAUNCH_CHECK(std::string(F8 ? "gemm_fp8" : "gemm_bf16"));
  return 0;
}

// 256x256 tiles (one workgroup per CU) once a launch has about two waves of
// them (500: a 100-tile product split 5 ways qualifies); 128x128 below
inline bool use_big_tile(const GemmArgs& a) {
  if (a.tile) return a.tile == 256;
  const long long big = (long long)((a.M + 255) / 256) * ((a.N + 255) / 256) * a.batch * a.k_split;
  return a.M >= 256 && a.N >= 256 && big >= 500;
}

template <bool AK, bool BKC, int EPI, int F8 = 0>
int launch_tiles(const GemmArgs& a, hipStream_t s) {
  if constexpr (EPI == EPI_QKV) {
    return launch_t<256, 256, AK, BKC, EPI, F8>(a, s);
  } else {
    if (use_big_tile(a)) return launch_t<256, 256, AK, BKC, EPI, F8>(a, s);
    return launch_t<128, 128, AK, BKC, EPI, F8>(a, s);
  }
}

}  // namespace
}  // namespace gs
