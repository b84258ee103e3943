// bf16 GEMM family on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Every dense contraction of the step runs here: the q/k/v, output, MLP and
// head projections of the model passage (dev.to "¿Cómo Entrenar Tu Propio
// ChatGPT por $50?", "1. Modelo GPT"; the bf16 cast of weights in
// "3. Gestión de Precisión"), their data and weight gradients, the chunked
// head/cross-entropy products, and the three products of each Newton-Schulz
// iteration ("2. Optimizador Muon": A = X^T X, B = b A + c A A, X = a X + X B).
//
// Design (gfx950):
//   * 256 threads = 4 waves in a 2x2 grid; workgroup tile BM x BN, K step 64.
//   * Operands are staged global -> registers -> LDS, double buffered, one
//     barrier per K step; the next step's global loads are in flight while the
//     current step's MFMAs run.
//   * LDS holds every operand tile k-contiguous (128 B per row, 16 B chunks
//     XOR-swizzled by row), which is the order MFMA fragments are read in.  An
//     operand that is contiguous along M/N in memory (the weight-gradient and
//     Gram products) is loaded as 8x8 blocks and transposed in registers
//     before the LDS write, so no product needs a transposed copy in HBM.
//   * The MFMA is issued with the operands swapped (B tile as src0), so each
//     lane's accumulators hold one output row and groups of 4 consecutive
//     columns: stores are 8/16-byte vectors and row reductions (the
//     cross-entropy epilogue) stay inside a lane pair.
//   * Workgroup ids are remapped so each of the 8 XCDs walks a contiguous
//     range of tiles, rasterised in groups of 8 row tiles for L2 reuse.

#pragma once

#include "common.h"
#include "gemm.h"

namespace gs {
namespace {

constexpr int kBK = 64;        // K elements per stage (128 bytes of bf16)
constexpr int kThreads = 256;

__device__ __forceinline__ int swz(int r) { return r & 7; }

// byte offset of 16-byte chunk kc of row r in a k-contiguous LDS tile
__device__ __forceinline__ int lds_off(int r, int kc) { return r * 128 + ((kc ^ swz(r)) << 4); }

// ---------------------------------------------------------------------------
// global -> register staging of one operand tile (R rows x 64 k)
// ---------------------------------------------------------------------------
template <int R, bool KC>
struct TileLoader {
  // k-contiguous: R*8 chunks of 16 B, R/32 per thread.
  // mn-contiguous: R*64/64 = R blocks of 8x8, one per thread (threads < R).
  static constexpr int kRegs = KC ? R / 32 : 8;
  uint4 v[kRegs];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, long long ld, int row0, int rows,
                                       int k0, int K, int tid) {
    const bool full = (row0 + R <= rows) && (k0 + kBK <= K);
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < kRegs; ++i) {
        const int c = tid + kThreads * i;
        const int r = c >> 3, kc = c & 7;
        const int gr = row0 + r, gk = k0 + kc * 8;
        if (full) {
          v[i] = *reinterpret_cast<const uint4*>(X + (long long)gr * ld + gk);
        } else {
          uint32_t w[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t lo = 0, hi = 0;
            if (gr < rows && gk + 2 * j < K) lo = X[(long long)gr * ld + gk + 2 * j];
            if (gr < rows && gk + 2 * j + 1 < K) hi = X[(long long)gr * ld + gk + 2 * j + 1];
            w[j] = lo | (hi << 16);
          }
          v[i] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    } else {
      if (tid < R) {
        const int rb = tid % (R / 8), kb = tid / (R / 8);
        const int gr = row0 + rb * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int gk = k0 + kb * 8 + j;
          if (full) {
            v[j] = *reinterpret_cast<const uint4*>(X + (long long)gk * ld + gr);
          } else {
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint32_t lo = 0, hi = 0;
              if (gk < K && gr + 2 * q < rows) lo = X[(long long)gk * ld + gr + 2 * q];
              if (gk < K && gr + 2 * q + 1 < rows) hi = X[(long long)gk * ld + gr + 2 * q + 1];
              w[q] = lo | (hi << 16);
            }
            v[j] = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
      }
    }
  }

  __device__ __forceinline__ void store(char* lds, int tid) const {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < kRegs; ++i) {
        const int c = tid + kThreads * i;
        const int r = c >> 3, kc = c & 7;
        *reinterpret_cast<uint4*>(lds + lds_off(r, kc)) = v[i];
      }
    } else {
      if (tid < R) {
        const int rb = tid % (R / 8), kb = tid / (R / 8);
        // v[j] holds k = kb*8 + j for rows rb*8 .. rb*8+7 (two rows per dword)
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const int d = rr >> 1;
          uint32_t w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t a = reinterpret_cast<const uint32_t*>(&v[2 * q])[d];
            const uint32_t b = reinterpret_cast<const uint32_t*>(&v[2 * q + 1])[d];
            w[q] = (rr & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
          }
          *reinterpret_cast<uint4*>(lds + lds_off(rb * 8 + rr, kb)) = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
  }
};

__device__ __forceinline__ bf16x8_t read_frag(const char* lds, int r, int kc) {
  return *reinterpret_cast<const bf16x8_t*>(lds + lds_off(r, kc));
}

// ---------------------------------------------------------------------------
// epilogues on 4 consecutive columns n .. n+3 of row m
// ---------------------------------------------------------------------------
template <int EPI>
__device__ __forceinline__ void epi4(const GemmArgs& p, int bi, int m, int n, const float* v) {
  const bool full = (n + 3 < p.N);
  if constexpr (EPI == EPI_F32 || EPI == EPI_RESID || EPI == EPI_F32_ATOMIC) {
    float* C = reinterpret_cast<float*>(p.C) + (long long)bi * p.sC + (long long)m * p.ldc + n;
    if (EPI == EPI_F32_ATOMIC) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n + j < p.N) unsafeAtomicAdd(C + j, v[j]);
    } else if (full) {
      float4 o = make_float4(v[0], v[1], v[2], v[3]);
      if (EPI == EPI_RESID || p.beta != 0.f) {
        const float4 c = *reinterpret_cast<const float4*>(C);
        const float b = (EPI == EPI_RESID) ? 1.f : p.beta;
        o.x += b * c.x; o.y += b * c.y; o.z += b * c.z; o.w += b * c.w;
      }
      *reinterpret_cast<float4*>(C) = o;
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
      if (full) {
        const uint2 w = *reinterpret_cast<const uint2*>(a);
        o[0] *= 2.f * sqrtf(lo_bf(w.x)); o[1] *= 2.f * sqrtf(hi_bf(w.x));
        o[2] *= 2.f * sqrtf(lo_bf(w.y)); o[3] *= 2.f * sqrtf(hi_bf(w.y));
      } else {
        for (int j = 0; j < 4; ++j) o[j] = (n + j < p.N) ? o[j] * 2.f * sqrtf(bf2f(a[j])) : 0.f;
      }
    }
    if constexpr (EPI == EPI_NS_POLY) {
      const float* a = reinterpret_cast<const float*>(p.aux) + (long long)bi * p.sAux + (long long)m * p.ldaux + n;
      for (int j = 0; j < 4; ++j) o[j] = (n + j < p.N) ? o[j] + p.beta * a[j] : 0.f;
    }
    if (full) {
      *reinterpret_cast<uint2*>(C) = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
    } else {
      for (int j = 0; j < 4; ++j)
        if (n + j < p.N) C[j] = f2bf(o[j]);
    }
  } else if constexpr (EPI == EPI_F32_BF16 || EPI == EPI_NS_UPD) {
    float* C = reinterpret_cast<float*>(p.C) + (long long)bi * p.sC + (long long)m * p.ldc + n;
    uint16_t* C2 = reinterpret_cast<uint16_t*>(p.C2) + (long long)bi * p.sC2 + (long long)m * p.ldc2 + n;
    float o[4];
    if (full) {
      o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
      if (EPI == EPI_NS_UPD) {
        const float4 c = *reinterpret_cast<const float4*>(C);
        o[0] += p.beta * c.x; o[1] += p.beta * c.y; o[2] += p.beta * c.z; o[3] += p.beta * c.w;
      }
      *reinterpret_cast<float4*>(C) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint2*>(C2) = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
    } else {
      for (int j = 0; j < 4; ++j)
        if (n + j < p.N) {
          float x = v[j];
          if (EPI == EPI_NS_UPD) x += p.beta * C[j];
          C[j] = x;
          C2[j] = f2bf(x);
        }
    }
  } else if constexpr (EPI == EPI_CE_BWD) {
    uint16_t* C = reinterpret_cast<uint16_t*>(p.C) + (long long)m * p.ldc + n;
    const int row_b = m / p.row_T, row_t = m - row_b * p.row_T;
    const int tgt = p.row_i[(long long)row_b * (p.row_T + 1) + row_t + 1] - p.col_offset;
    const float lse = p.row_f[m];
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // v already carries alpha = 1; the 1/(B*T) factor is in beta
      o[j] = (__expf(v[j] - lse) - ((n + j) == tgt ? 1.f : 0.f)) * p.beta;
    }
    if (full) {
      *reinterpret_cast<uint2*>(C) = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
    } else {
      for (int j = 0; j < 4; ++j)
        if (n + j < p.N) C[j] = f2bf(o[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int BM, int BN, bool AK, bool BKC, int EPI>
__global__ void __launch_bounds__(kThreads, 1) gemm_bf16_kernel(GemmArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  constexpr int GM = 8;
  const int group = lid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in_group = lid - group * GM * tiles_n;
  const int tile_m = first_m + in_group % gsz;
  const int tile_n = in_group / gsz;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  const int bi = blockIdx.y / p.k_split, split = blockIdx.y % p.k_split;
  const int nk_all = (p.K + kBK - 1) / kBK;
  const int nk_per = (nk_all + p.k_split - 1) / p.k_split;
  const int kt0 = split * nk_per;
  const int nk = max(0, min(nk_all, kt0 + nk_per) - kt0);

  const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A) + (long long)bi * p.sA;
  const uint16_t* B = reinterpret_cast<const uint16_t*>(p.B) + (long long)bi * p.sB;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  TileLoader<BM, AK> la;
  TileLoader<BN, BKC> lb;
  if (nk > 0) {
    la.load(A, p.lda, m0, p.M, kt0 * kBK, p.K, tid);
    lb.load(B, p.ldb, n0, p.N, kt0 * kBK, p.K, tid);
    la.store(smem, tid);
    lb.store(smem + A_BYTES, tid);
  }
  __syncthreads();

  const int lr = lane & 31, lh = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const char* sa = smem + (kt & 1) * STAGE;
    const char* sb = sa + A_BYTES;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(A, p.lda, m0, p.M, (kt0 + kt + 1) * kBK, p.K, tid);
      lb.load(B, p.ldb, n0, p.N, (kt0 + kt + 1) * kBK, p.K, tid);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8_t fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = read_frag(sa, wm * WM + i * 32 + lr, ks * 2 + lh);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = read_frag(sb, wn * WN + j * 32 + lr, ks * 2 + lh);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      char* nxt = smem + ((kt + 1) & 1) * STAGE;
      la.store(nxt, tid);
      lb.store(nxt + A_BYTES, tid);
    }
    __syncthreads();
  }

  // ----------------------------- epilogue ---------------------------------
  if constexpr (EPI == EPI_QKV) {
    // Each wave owns 128 columns = one head (tiles are 256 wide).  Lane row m
    // holds head features e = j*32 + 8g + 4lh + r; the rotation partner
    // e + 64 sits in the same lane at j + 2, the other half of the head in
    // lane ^ 32.
    static_assert(WN == 128, "EPI_QKV needs 128 columns per wave");
    const int nb = n0 + wn * WN;        // first column of this wave's head
    const int dmodel = p.n_head * 128;
    const bool is_qk = nb < 2 * dmodel;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm * WM + i * 32 + lr;
      float y[TN][16];
      float ss = 0.f;
      const int t = (m < p.M) ? m % p.row_T : 0;
      if (is_qk) {
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
              const float x1 = acc[i][j][4 * g + r] * p.alpha, x2 = acc[i][j + 2][4 * g + r] * p.alpha;
              const float y1 = x1 * cc[r] - x2 * sn[r], y2 = x1 * sn[r] + x2 * cc[r];
              y[j][4 * g + r] = y1;
              y[j + 2][4 * g + r] = y2;
              ss += y1 * y1 + y2 * y2;
            }
          }
        ss += __shfl_xor(ss, 32, 64);
        const float rr = 1.0f / sqrtf(ss / 128.f + 1e-6f);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) y[j][e] *= rr;
        if (lh == 0 && m < p.M) {
          const int head = (nb % dmodel) / 128;
          float* rdst = (nb < dmodel) ? p.part : p.zt;
          rdst[(long long)m * p.n_head + head] = rr;
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) y[j][e] = acc[i][j][e] * p.alpha;
      }
      if (m >= p.M || nb >= p.N) continue;
      uint16_t* crow = reinterpret_cast<uint16_t*>(p.C) + (long long)m * p.ldc + nb;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int e = j * 32 + 8 * g + 4 * lh;
          *reinterpret_cast<uint2*>(crow + e) = make_uint2(pack_bf2(y[j][4 * g], y[j][4 * g + 1]),
                                                           pack_bf2(y[j][4 * g + 2], y[j][4 * g + 3]));
        }
    }
  } else if constexpr (EPI == EPI_CE_FWD) {
    // Per row: max and sum of exp over this wave's WN columns, merged with
    // the partner lane (lane ^ 32) that holds the other half of the columns.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm * WM + i * 32 + lr;
      int tgt = -1;
      if (m < p.M) {
        const int row_b = m / p.row_T, row_t = m - row_b * p.row_T;
        tgt = p.row_i[(long long)row_b * (p.row_T + 1) + row_t + 1] - p.col_offset;
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
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int n = n0 + wn * WN + j * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
          if (n < p.N) s += __expf(acc[i][j][e] * p.alpha - mx);
        }
      s += __shfl_xor(s, 32, 64);
      if (lh == 0 && m < p.M && n0 + wn * WN < p.N) {
        reinterpret_cast<float2*>(p.part)[(long long)m * p.nparts + tile_n * 2 + wn] = make_float2(mx, s);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm * WM + i * 32 + lr;
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN + j * 32 + 8 * g + 4 * lh;
          if (n >= p.N) continue;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * g + r] * p.alpha;
          epi4<EPI>(p, bi, m, n, v);
        }
    }
  }
}

template <int BM, int BN, bool AK, bool BKC, int EPI>
int launch_t(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  dim3 grid(tiles, a.batch * a.k_split);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, AK, BKC, EPI>), grid, dim3(kThreads), 0, s, a);
  GS_LAUNCH_CHECK("gemm_bf16");
  return 0;
}

inline bool use_big_tile(const GemmArgs& a) {
  const long long big = (long long)((a.M + 255) / 256) * ((a.N + 255) / 256) * a.batch * a.k_split;
  return a.M >= 256 && a.N >= 256 && big >= 512;
}

template <bool AK, bool BKC, int EPI>
int launch_tiles(const GemmArgs& a, hipStream_t s) {
  if constexpr (EPI == EPI_QKV) {
    return launch_t<256, 256, AK, BKC, EPI>(a, s);
  } else {
    if (use_big_tile(a)) return launch_t<256, 256, AK, BKC, EPI>(a, s);
    return launch_t<128, 128, AK, BKC, EPI>(a, s);
  }
}

}  // namespace
}  // namespace gs
