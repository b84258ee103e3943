// Internal interface of the bf16 / fp8 GEMM family of libgptstep.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gs {

// Epilogues fused into the GEMM (v = alpha * sum_k A[m,k] B[n,k]):
enum Epi {
  EPI_F32 = 0,     // C f32 = v + beta * C
  EPI_BF16,        // C bf16 = v
  EPI_RESID,       // C f32 += v (residual stream add; one writer per element)
  EPI_RELU2,       // C bf16 = max(v, 0)^2
  EPI_DRELU2,      // C bf16 = v * 2 sqrt(aux_bf16)       (ReLU^2 backward from a = relu(u)^2)
  EPI_NS_POLY,     // C bf16 = beta * aux_bf16 + v        (B = b A + c A A, alpha = c, beta = b;
                   // and X = a X + X B with aux = X, beta = a)
  EPI_CE_FWD,      // per-row partial (max mx, sum exp) over each wave's columns + target logit;
                   // with C given, also C fp16 = exp(v - mx), kept for the backward
  EPI_F16,         // C fp16 = v (the stored exponentials of EPI_CE_FWD; not launched alone)
  EPI_QKV,         // [q | k | v] projection: rotate + RMS-normalise each 128-wide q/k head,
                   // C bf16; per (row, head) 1/rms to rq / rk (part, zt); needs 256-wide tiles
  EPI_COUNT
};

// C[b][m, n] = epilogue(alpha * sum_k A[b][m, k] * B[b][n, k]) for b < batch.
// Operand layout: k-contiguous means element (r, k) at X[r * ld + k];
// mn-contiguous means element (r, k) at X[k * ld + r].
struct GemmArgs {
  int M = 0, N = 0, K = 0, batch = 1;
  const void* A = nullptr; long long lda = 0, sA = 0; int a_kcontig = 1;
  const void* B = nullptr; long long ldb = 0, sB = 0; int b_kcontig = 1;
  void* C = nullptr; long long ldc = 0, sC = 0;
  void* C2 = nullptr; long long ldc2 = 0, sC2 = 0;
  const void* aux = nullptr; long long ldaux = 0, sAux = 0;
  float alpha = 1.f, beta = 0.f;
  const float* row_f = nullptr;  // per-row float (lse)
  const int* row_i = nullptr;    // per-row int (target ids), element m at row_i[(m / T) * (T+1) + m % T + 1]
  int row_T = 1;                 // T used for the target indexing above
  int col_offset = 0;            // global column of n = 0 (vocab chunking)
  float* part = nullptr;         // CE partials: float2 [M, nparts]
  int nparts = 0;
  float* zt = nullptr;           // CE target logit [M]
  int k_split = 1;               // > 1: EPI_F32 writing one partial per split
  long long split_stride = 0;    // EPI_F32 with k_split > 1: split s writes C + s * split_stride
  const float* rope = nullptr;    // EPI_QKV: cos [row_T, 64] then sin [row_T, 64]
  int n_head = 0;                 // EPI_QKV: query heads
  int n_kv_head = 0;              // EPI_QKV: key/value heads (0 = n_head); columns [q | k | v]
  const float* scale_a = nullptr;  // fp8: device scalars; v *= 1 / (scale_a * scale_b)
  const float* scale_b = nullptr;
  int sym = 0;                     // M == N, symmetric product: only tiles with tile_m <= tile_n are
                                   // computed; the caller fills the rest (launch_sym_mirror)
  int tile = 0;                    // 0: tile chosen from the sizes; 128 or 256 forces that tile
                                   // (launches that must agree on their column groups)
  float* amax = nullptr;           // bf16 epilogues: per-wave max |stored value| at
                                   // amax[block * waves + wave] (block = x + gridDim.x * y)
};

// Tile selection visible to callers that size partial buffers.
int gemm_tile_n(const GemmArgs& a);
// Number of per-wave amax partials a launch with these arguments writes.
long long gemm_amax_slots(const GemmArgs& a);

// Launch; returns 0 or the gpt_status error code.
int gemm_bf16(const GemmArgs& a, int epi, hipStream_t s);
// fp8 (both operands k-contiguous, 1-byte codes; fmt 0 = E4M3, 1 = E5M2).
int gemm_fp8(const GemmArgs& a, int epi, int fmt_a, int fmt_b, hipStream_t s);

}  // namespace gs
