// Causal flash attention forward and backward, head width 128, on CDNA4
// matrix cores (v_mfma_f32_32x32x16_bf16).
//
// The model passage (dev.to "¿Cómo Entrenar Tu Propio ChatGPT por $50?",
// "1. Modelo GPT" and "5. Unificación Flash Attention") calls
// flash_attn_func(q, k, v, causal=True): y_t = sum_{j<=t} softmax_j(q_t.k_j /
// sqrt(128)) v_j, with the row statistics kept (online softmax) instead of the
// T x T score matrix.
//
// Forward (one workgroup = 128 queries of one (batch, head), 4 waves x 32):
//   * the wave computes S^T = K Q^T, so in the accumulator layout each lane
//     owns ONE query and 32 of the tile's keys (its partner lane, lane ^ 32,
//     owns the other 32): the row max needs one cross-lane swap per tile and
//     the row sum none until the end;
//   * O^T = V^T P^T uses P straight from the accumulators as the B operand;
//     the order of keys inside a k-step is the accumulator order, and V^T is
//     read from LDS in that same order (it is stored transposed, keys
//     contiguous, by an 8x8 register transpose at load time);
//   * K / V tiles of 64 keys are double buffered in LDS.
// Backward, two kernels and no atomics:
//   * dK/dV: one workgroup = 128 keys (4 waves x 32 keys) looping over query
//     tiles of 32: recompute S = Q K^T and P = exp(S - lse), dP = dO V^T,
//     dS = P (dP - delta), then dV^T += dO^T P and dK^T += Q^T dS with P and
//     dS taken straight from the accumulators;
//   * dQ: one workgroup = 128 queries looping over key tiles of 64, shaped
//     like the forward: S^T and dP^T recomputed, dQ^T += K^T dS^T.
// The second kernel recomputes two of the four products of the first; in
// exchange dQ needs neither fp32 atomics nor a pass through LDS for dS, and
// the result is deterministic.

#include "common.h"
#include "kernels.h"

namespace gs {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;  // log2 of the largest unnormalised P

__device__ __forceinline__ int sw(int r) { return r & 7; }
// rows of 256 bytes (16 chunks of 16 B)
__device__ __forceinline__ int off256(int r, int c) { return r * 256 + ((c ^ sw(r)) << 4); }
// rows of 128 bytes (8 chunks of 16 B)
__device__ __forceinline__ int off128(int r, int c) { return r * 128 + ((c ^ sw(r)) << 4); }

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// column c of an 8x8 bf16 block held as 8 rows of 16 B
__device__ __forceinline__ uint4 column8x8(const uint4* in, int c) {
  const int d = c >> 1;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a = reinterpret_cast<const uint32_t*>(&in[2 * q])[d];
    const uint32_t b = reinterpret_cast<const uint32_t*>(&in[2 * q + 1])[d];
    w[q] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// column c of an 8x4 bf16 block held as 8 rows of 8 B
__device__ __forceinline__ uint4 column8x4(const uint2* in, int c) {
  const int d = c >> 1;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a = reinterpret_cast<const uint32_t*>(&in[2 * q])[d];
    const uint32_t b = reinterpret_cast<const uint32_t*>(&in[2 * q + 1])[d];
    w[q] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// B/A fragment of 8 keys in accumulator order from a transposed tile
// (row = feature, keys contiguous): keys 16s+4h+0..3 and 16s+8+4h+0..3.
__device__ __forceinline__ bf16x8_t read_perm_frag(const char* lds, int row, int s, int h) {
  const uint2 a = *reinterpret_cast<const uint2*>(lds + off128(row, 2 * s) + 8 * h);
  const uint2 b = *reinterpret_cast<const uint2*>(lds + off128(row, 2 * s + 1) + 8 * h);
  bf16x8_t f;
  uint32_t* w = reinterpret_cast<uint32_t*>(&f);
  w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y;
  return f;
}

// pack accumulator values {4g0 .. 4g0+3, 4g1 .. 4g1+3} of x as bf16 (k-step s)
__device__ __forceinline__ bf16x8_t pack_perm(const float* x, int s) {
  bf16x8_t f;
  uint32_t* w = reinterpret_cast<uint32_t*>(&f);
  const int g0 = 8 * s;  // values 4*(2s) .. 4*(2s)+7
  w[0] = pack_bf2(x[g0 + 0], x[g0 + 1]);
  w[1] = pack_bf2(x[g0 + 2], x[g0 + 3]);
  w[2] = pack_bf2(x[g0 + 4], x[g0 + 5]);
  w[3] = pack_bf2(x[g0 + 6], x[g0 + 7]);
  return f;
}

// ============================================================================
// forward
// ============================================================================
constexpr int FQ = 128;  // queries per workgroup
constexpr int FK = 64;   // keys per tile

struct KVLoad {
  uint4 k[4];  // 4 chunks of K: rows (t + 256 i) / 16, chunk % 16
  uint4 v[8];  // one 8x8 block of V (threads < 128)
};

__device__ __forceinline__ void fwd_load_kv(KVLoad& L, const uint16_t* kbase, const uint16_t* vbase,
                                            long long ld, int key0, int T, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 4, ch = c & 15;
    const int key = key0 + r;
    L.k[i] = key < T ? ld16(kbase + (long long)key * ld + ch * 8) : make_uint4(0, 0, 0, 0);
  }
  if (tid < 128) {
    const int kb = tid & 7, eb = tid >> 3;  // keys kb*8.., features eb*8..
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = key0 + kb * 8 + j;
      L.v[j] = key < T ? ld16(vbase + (long long)key * ld + eb * 8) : make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void fwd_store_kv(const KVLoad& L, char* sk, char* svt, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 4, ch = c & 15;
    *reinterpret_cast<uint4*>(sk + off256(r, ch)) = L.k[i];
  }
  if (tid < 128) {
    const int kb = tid & 7, eb = tid >> 3;
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4*>(svt + off128(eb * 8 + c, kb)) = column8x8(L.v, c);
  }
}

__global__ void __launch_bounds__(256, 2)
attn_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                long long ld, uint16_t* __restrict__ out, long long ld_out, float* __restrict__ lse, int H, int T) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (FK * 256 + 128 * 128)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int nqb = (T + FQ - 1) / FQ;
  const int qb = nqb - 1 - blockIdx.x;  // longest rows first
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const long long rowbase = (long long)b * T;
  const uint16_t* qh = q + rowbase * ld + h * 128;
  const uint16_t* kh = k + rowbase * ld + h * 128;
  const uint16_t* vh = v + rowbase * ld + h * 128;

  const int q0 = qb * FQ;
  const int wq0 = q0 + wave * 32;   // first query of this wave
  const int myq = wq0 + lr;         // this lane's query
  const float c = 0.08838834764831845f * kLog2e;  // 1/sqrt(128) in log2 units

  // Q fragments (B operand: column = query, 8 features per k-step)
  bf16x8_t fq[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (myq < T) {
      const uint4 w = ld16(qh + (long long)myq * ld + ks * 16 + lh * 8);
      fq[ks] = *reinterpret_cast<const bf16x8_t*>(&w);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) fq[ks][e] = 0;
    }
  }

  f32x16_t o[4];
#pragma unroll
  for (int et = 0; et < 4; ++et)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[et][e] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int last_key = min(T - 1, q0 + FQ - 1);
  const int ntiles = last_key / FK + 1;
  constexpr int STAGE = FK * 256 + 128 * 128;

  KVLoad L;
  fwd_load_kv(L, kh, vh, ld, 0, T, tid);
  fwd_store_kv(L, smem, smem + FK * 256, tid);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const char* sk = smem + (j & 1) * STAGE;
    const char* svt = sk + FK * 256;
    const bool more = j + 1 < ntiles;
    if (more) fwd_load_kv(L, kh, vh, ld, (j + 1) * FK, T, tid);

    const int key0 = j * FK;
    // wave-uniform: skip the tile when every key is after this wave's queries
    if (key0 <= wq0 + 31) {
      f32x16_t s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8_t fk = *reinterpret_cast<const bf16x8_t*>(sk + off256(kt * 32 + lr, ks * 2 + lh));
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk, fq[ks], s[kt], 0, 0, 0);
        }
      }
      // scale, mask (diagonal / ragged tiles only), tile max
      const bool diag = (key0 + FK - 1 > wq0) || (key0 + FK > T);  // wave-uniform
      float x[32];
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float val = s[kt][e] * c;
          if (diag) {
            const int key = key0 + kt * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
            val = (key <= myq && key < T) ? val : -INFINITY;
          }
          x[kt * 16 + e] = val;
          tmax = fmaxf(tmax, val);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      // lazy rescale: the reference max moves only when a row max exceeds it
      // by more than 2^8, so P stays <= 256 and most tiles skip the O rescale
      const bool need = tmax > m + kRescale;
      if (__any(need)) {
        const float mn = need ? tmax : m;
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        l *= alpha;
        m = mn;
#pragma unroll
        for (int et = 0; et < 4; ++et)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[et][e] *= alpha;
      }
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        x[i] = __builtin_amdgcn_exp2f(x[i] - m);
        psum += x[i];
      }
      l += psum;
      // O^T += V^T P^T over the 64 keys (4 k-steps of 16)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8_t fp = pack_perm(x + (st >> 1) * 16, st & 1);
#pragma unroll
        for (int et = 0; et < 4; ++et) {
          const bf16x8_t fv = read_perm_frag(svt, et * 32 + lr, st, lh);
          o[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv, fp, o[et], 0, 0, 0);
        }
      }
    }
    if (more) {
      char* nk = smem + ((j + 1) & 1) * STAGE;
      fwd_store_kv(L, nk, nk + FK * 256, tid);
    }
    __syncthreads();
  }

  l += __shfl_xor(l, 32, 64);
  if (myq < T) {
    const float inv = 1.f / l;
    uint16_t* orow = out + (rowbase + myq) * ld_out + h * 128;
#pragma unroll
    for (int et = 0; et < 4; ++et)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = et * 32 + 8 * g + 4 * lh;
        *reinterpret_cast<uint2*>(orow + e) =
            make_uint2(pack_bf2(o[et][4 * g] * inv, o[et][4 * g + 1] * inv),
                       pack_bf2(o[et][4 * g + 2] * inv, o[et][4 * g + 3] * inv));
      }
    if (lh == 0) lse[(long long)bh * T + myq] = m * kLn2 + logf(l);
  }
}

// ============================================================================
// backward
// ============================================================================
// delta[b,h,t] = sum_e dout * out.  One wave per (token, head).
__global__ void __launch_bounds__(256) attn_bwd_pre_kernel(const uint16_t* __restrict__ out,
                                                           const uint16_t* __restrict__ dout, long long ld_out,
                                                           float* __restrict__ delta, int H, int T, long long NH) {
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= NH) return;
  const long long n = w / H;
  const int h = (int)(w % H);
  const uint32_t ow = reinterpret_cast<const uint32_t*>(out + n * ld_out + h * 128)[lane];
  const uint32_t dw = reinterpret_cast<const uint32_t*>(dout + n * ld_out + h * 128)[lane];
  const float s = wave_sum(lo_bf(ow) * lo_bf(dw) + hi_bf(ow) * hi_bf(dw));
  const long long b = n / T, t = n % T;
  if (lane == 0) delta[(b * H + h) * T + t] = s;
}

// rows of 64 bytes (4 chunks of 16 B)
__device__ __forceinline__ int off64(int r, int c) { return r * 64 + ((c ^ (r & 3)) << 4); }

__device__ __forceinline__ bf16x8_t read_perm_frag64(const char* lds, int row, int s, int h) {
  const uint2 a = *reinterpret_cast<const uint2*>(lds + off64(row, 2 * s) + 8 * h);
  const uint2 b = *reinterpret_cast<const uint2*>(lds + off64(row, 2 * s + 1) + 8 * h);
  bf16x8_t f;
  uint32_t* w = reinterpret_cast<uint32_t*>(&f);
  w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y;
  return f;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup = 128 keys (4 waves x 32), query tiles of 32.
//   S = Q K^T, dP = dO V^T (accumulator: column = key, rows = queries)
//   P = exp(S - lse), dS = P (dP - delta)
//   dV^T += dO^T P, dK^T += Q^T dS  (P, dS as B operands in accumulator order)
// ---------------------------------------------------------------------------
constexpr int KV_KEYS = 128;
constexpr int KV_Q = 32;
constexpr int KV_SK = 0;                          // K natural [128 keys][256 B]
constexpr int KV_QN = KV_SK + KV_KEYS * 256;      // Q natural [32][256 B]
constexpr int KV_QT = KV_QN + KV_Q * 256;         // Q^T [128 e][64 B]
constexpr int KV_DN = KV_QT + 128 * 64;           // dO natural
constexpr int KV_DT = KV_DN + KV_Q * 256;         // dO^T
constexpr int KV_LSE = KV_DT + 128 * 64;          // lse * log2e [32]
constexpr int KV_DEL = KV_LSE + KV_Q * 4;         // delta [32]
constexpr int KV_TOTAL = KV_DEL + KV_Q * 4;

__global__ void __launch_bounds__(256, 2)
attn_bwd_kv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                   long long ld, const uint16_t* __restrict__ dout, long long ld_out, const float* __restrict__ lse,
                   const float* __restrict__ delta, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                   long long ld_dkv, int H, int T) {
  __shared__ __attribute__((aligned(16))) char smem[KV_TOTAL];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int kb = blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const long long rowbase = (long long)b * T;
  const uint16_t* qh = q + rowbase * ld + h * 128;
  const uint16_t* kh = k + rowbase * ld + h * 128;
  const uint16_t* vh = v + rowbase * ld + h * 128;
  const uint16_t* doh = dout + rowbase * ld_out + h * 128;
  const float* lseh = lse + (long long)bh * T;
  const float* delh = delta + (long long)bh * T;
  const float scale = 0.08838834764831845f;
  const float c = scale * kLog2e;

  const int k0 = kb * KV_KEYS;
  const int wk0 = k0 + wave * 32;
  const int mykey = wk0 + lr;

  // V fragments of the wave's keys (B operand: column = key, 8 features per k-step)
  bf16x8_t fv[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (mykey < T) {
      const uint4 a = ld16(vh + (long long)mykey * ld + ks * 16 + lh * 8);
      fv[ks] = *reinterpret_cast<const bf16x8_t*>(&a);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) fv[ks][e] = 0;
    }
  }
  // K of the whole block in LDS
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int cidx = tid + 256 * i;
    const int r = cidx >> 4, ch = cidx & 15;
    const int key = k0 + r;
    *reinterpret_cast<uint4*>(smem + KV_SK + off256(r, ch)) =
        key < T ? ld16(kh + (long long)key * ld + ch * 8) : make_uint4(0, 0, 0, 0);
  }

  f32x16_t dvt[4], dkt[4];
#pragma unroll
  for (int et = 0; et < 4; ++et)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dvt[et][e] = 0.f; dkt[et][e] = 0.f; }

  const int nqt = (T + KV_Q - 1) / KV_Q;
  for (int qt = k0 / KV_Q; qt < nqt; ++qt) {
    const int q0 = qt * KV_Q;
    __syncthreads();
    {
      // an 8x4 block of Q (tid < 128) or dO: queries qb*8 .. +7, features eb*4 .. +3
      const int blk = tid & 127, qb = blk & 3, eb = blk >> 2;
      const bool isq = tid < 128;
      const uint16_t* base = isq ? qh : doh;
      const long long ldx = isq ? ld : ld_out;
      uint2 r8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int qq = q0 + qb * 8 + j;
        r8[j] = qq < T ? *reinterpret_cast<const uint2*>(base + (long long)qq * ldx + eb * 4) : make_uint2(0, 0);
      }
      char* nat = smem + (isq ? KV_QN : KV_DN);
      char* tr = smem + (isq ? KV_QT : KV_DT);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint2*>(nat + off256(qb * 8 + j, eb >> 1) + 8 * (eb & 1)) = r8[j];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) *reinterpret_cast<uint4*>(tr + off64(eb * 4 + cc, qb)) = column8x4(r8, cc);
      if (tid < KV_Q) {
        const int qq = q0 + tid;
        reinterpret_cast<float*>(smem + KV_LSE)[tid] = qq < T ? lseh[qq] * kLog2e : INFINITY;
      } else if (tid < 2 * KV_Q) {
        const int i = tid - KV_Q, qq = q0 + i;
        reinterpret_cast<float*>(smem + KV_DEL)[i] = qq < T ? delh[qq] : 0.f;
      }
    }
    __syncthreads();
    if (q0 + KV_Q - 1 < wk0) continue;  // every query of the tile precedes every key of the wave

    f32x16_t sacc, dpacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) { sacc[e] = 0.f; dpacc[e] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t aq = *reinterpret_cast<const bf16x8_t*>(smem + KV_QN + off256(lr, ks * 2 + lh));
      const bf16x8_t bk = *reinterpret_cast<const bf16x8_t*>(smem + KV_SK + off256(wave * 32 + lr, ks * 2 + lh));
      const bf16x8_t ad = *reinterpret_cast<const bf16x8_t*>(smem + KV_DN + off256(lr, ks * 2 + lh));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bk, sacc, 0, 0, 0);
      dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, fv[ks], dpacc, 0, 0, 0);
    }
    const float* slse = reinterpret_cast<const float*>(smem + KV_LSE);
    const float* sdel = reinterpret_cast<const float*>(smem + KV_DEL);
    const bool diag = (q0 < wk0 + 31) || (q0 + KV_Q > T) || (wk0 + 32 > T);
    // P and dS packed to bf16 straight away, in accumulator order (k-step st
    // holds values 8 st .. 8 st + 7)
    bf16x8_t fp[2], fs[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      uint32_t* wp = reinterpret_cast<uint32_t*>(&fp[st]);
      uint32_t* wd = reinterpret_cast<uint32_t*>(&fs[st]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float pv[2], dv2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = 8 * st + 2 * i + u;
          const int ql = 8 * (e >> 2) + 4 * lh + (e & 3);
          float pe = __builtin_amdgcn_exp2f(sacc[e] * c - slse[ql]);
          if (diag) pe = (mykey <= q0 + ql && mykey < T) ? pe : 0.f;
          pv[u] = pe;
          dv2[u] = pe * (dpacc[e] - sdel[ql]);
        }
        wp[i] = pack_bf2(pv[0], pv[1]);
        wd[i] = pack_bf2(dv2[0], dv2[1]);
      }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int et = 0; et < 4; ++et) {
        const bf16x8_t ad = read_perm_frag64(smem + KV_DT, et * 32 + lr, st, lh);
        const bf16x8_t aq = read_perm_frag64(smem + KV_QT, et * 32 + lr, st, lh);
        dvt[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, fp[st], dvt[et], 0, 0, 0);
        dkt[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, fs[st], dkt[et], 0, 0, 0);
      }
    }
  }

  if (mykey < T) {
    uint16_t* dkr = dk + (rowbase + mykey) * ld_dkv + h * 128;
    uint16_t* dvr = dv + (rowbase + mykey) * ld_dkv + h * 128;
#pragma unroll
    for (int et = 0; et < 4; ++et)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = et * 32 + 8 * g + 4 * lh;
        *reinterpret_cast<uint2*>(dkr + e) =
            make_uint2(pack_bf2(dkt[et][4 * g] * scale, dkt[et][4 * g + 1] * scale),
                       pack_bf2(dkt[et][4 * g + 2] * scale, dkt[et][4 * g + 3] * scale));
        *reinterpret_cast<uint2*>(dvr + e) =
            make_uint2(pack_bf2(dvt[et][4 * g], dvt[et][4 * g + 1]), pack_bf2(dvt[et][4 * g + 2], dvt[et][4 * g + 3]));
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup = 128 queries (4 waves x 32), key tiles of 64.
//   S^T = K Q^T, dP^T = V dO^T (accumulator: column = query, rows = keys)
//   dS^T = P^T (dP^T - delta);  dQ^T += K^T dS^T  (dS^T as B operand)
// ---------------------------------------------------------------------------
constexpr int DQ_Q = 128;
constexpr int DQ_K = 64;
constexpr int DQ_KN = 0;                       // K natural [64][256 B]
constexpr int DQ_VN = DQ_KN + DQ_K * 256;      // V natural [64][256 B]
constexpr int DQ_KT = DQ_VN + DQ_K * 256;      // K^T [128 e][128 B]
constexpr int DQ_TOTAL = DQ_KT + 128 * 128;

__global__ void __launch_bounds__(256, 2)
attn_bwd_q_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                  long long ld, const uint16_t* __restrict__ dout, long long ld_out, const float* __restrict__ lse,
                  const float* __restrict__ delta, float* __restrict__ dq_out, int H, int T) {
  __shared__ __attribute__((aligned(16))) char smem[DQ_TOTAL];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int nqb = (T + DQ_Q - 1) / DQ_Q;
  const int qb = nqb - 1 - blockIdx.x;  // longest rows first
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const long long rowbase = (long long)b * T;
  const int d = H * 128;
  const uint16_t* qh = q + rowbase * ld + h * 128;
  const uint16_t* kh = k + rowbase * ld + h * 128;
  const uint16_t* vh = v + rowbase * ld + h * 128;
  const uint16_t* doh = dout + rowbase * ld_out + h * 128;
  const float scale = 0.08838834764831845f;
  const float c = scale * kLog2e;

  const int q0 = qb * DQ_Q;
  const int wq0 = q0 + wave * 32;
  const int myq = wq0 + lr;
  bf16x8_t fq[8], fd[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (myq < T) {
      const uint4 a = ld16(qh + (long long)myq * ld + ks * 16 + lh * 8);
      const uint4 bq = ld16(doh + (long long)myq * ld_out + ks * 16 + lh * 8);
      fq[ks] = *reinterpret_cast<const bf16x8_t*>(&a);
      fd[ks] = *reinterpret_cast<const bf16x8_t*>(&bq);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { fq[ks][e] = 0; fd[ks][e] = 0; }
    }
  }
  const float lse2 = myq < T ? lse[(long long)bh * T + myq] * kLog2e : INFINITY;
  const float del = myq < T ? delta[(long long)bh * T + myq] : 0.f;

  f32x16_t dqt[4];
#pragma unroll
  for (int et = 0; et < 4; ++et)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqt[et][e] = 0.f;

  const int last_key = min(T - 1, q0 + DQ_Q - 1);
  const int ntiles = last_key / DQ_K + 1;
  for (int j = 0; j < ntiles; ++j) {
    const int key0 = j * DQ_K;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cidx = tid + 256 * i;
      const int r = cidx >> 4, ch = cidx & 15;
      const int key = key0 + r;
      const bool ok = key < T;
      *reinterpret_cast<uint4*>(smem + DQ_KN + off256(r, ch)) =
          ok ? ld16(kh + (long long)key * ld + ch * 8) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(smem + DQ_VN + off256(r, ch)) =
          ok ? ld16(vh + (long long)key * ld + ch * 8) : make_uint4(0, 0, 0, 0);
    }
    if (tid < 128) {
      const int kb8 = tid & 7, eb = tid >> 3;
      uint4 r8[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int key = key0 + kb8 * 8 + jj;
        r8[jj] = key < T ? ld16(kh + (long long)key * ld + eb * 8) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
        *reinterpret_cast<uint4*>(smem + DQ_KT + off128(eb * 8 + cc, kb8)) = column8x8(r8, cc);
    }
    __syncthreads();
    if (key0 > wq0 + 31) continue;  // wave-uniform: every key follows every query of the wave

    f32x16_t st[2], dpt[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) { st[kt][e] = 0.f; dpt[kt][e] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t ak = *reinterpret_cast<const bf16x8_t*>(smem + DQ_KN + off256(kt * 32 + lr, ks * 2 + lh));
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(smem + DQ_VN + off256(kt * 32 + lr, ks * 2 + lh));
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, fq[ks], st[kt], 0, 0, 0);
        dpt[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, fd[ks], dpt[kt], 0, 0, 0);
      }
    }
    const bool diag = (key0 + DQ_K - 1 > wq0) || (key0 + DQ_K > T);
    float ds[32];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = key0 + kt * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
        float pv = __builtin_amdgcn_exp2f(st[kt][e] * c - lse2);
        if (diag) pv = (key <= myq && key < T) ? pv : 0.f;
        ds[kt * 16 + e] = pv * (dpt[kt][e] - del);
      }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const bf16x8_t fs = pack_perm(ds + (s4 >> 1) * 16, s4 & 1);
#pragma unroll
      for (int et = 0; et < 4; ++et) {
        const bf16x8_t ak = read_perm_frag(smem + DQ_KT, et * 32 + lr, s4, lh);
        dqt[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, fs, dqt[et], 0, 0, 0);
      }
    }
  }
  if (myq < T) {
    float* dqr = dq_out + (rowbase + myq) * d + h * 128;
#pragma unroll
    for (int et = 0; et < 4; ++et)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = et * 32 + 8 * g + 4 * lh;
        *reinterpret_cast<float4*>(dqr + e) = make_float4(dqt[et][4 * g] * scale, dqt[et][4 * g + 1] * scale,
                                                          dqt[et][4 * g + 2] * scale, dqt[et][4 * g + 3] * scale);
      }
  }
}

}  // namespace

int launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, long long ld_qkv, uint16_t* out,
                    long long ld_out, float* lse, int B, int H, int T, hipStream_t s) {
  if (B <= 0 || T <= 0) return 0;
  dim3 grid((T + FQ - 1) / FQ, B * H);
  hipLaunchKernelGGL(attn_fwd_kernel, grid, dim3(256), 0, s, q, k, v, ld_qkv, out, ld_out, lse, H, T);
  GS_LAUNCH_CHECK("attn_fwd");
  return 0;
}

int launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, long long ld_qkv,
                    const uint16_t* out, const uint16_t* dout, long long ld_out, const float* lse, float* delta,
                    float* dq, uint16_t* dk, uint16_t* dv, long long ld_dkv, int B, int H, int T,
                    hipStream_t s) {
  if (B <= 0 || T <= 0) return 0;
  const long long NH = (long long)B * T * H;
  hipLaunchKernelGGL(attn_bwd_pre_kernel, dim3((unsigned)((NH + 3) / 4)), dim3(256), 0, s, out, dout, ld_out,
                     delta, H, T, NH);
  GS_LAUNCH_CHECK("attn_bwd_pre");
  hipLaunchKernelGGL(attn_bwd_kv_kernel, dim3((T + KV_KEYS - 1) / KV_KEYS, B * H), dim3(256), 0, s, q, k, v,
                     ld_qkv, dout, ld_out, lse, delta, dk, dv, ld_dkv, H, T);
  GS_LAUNCH_CHECK("attn_bwd_kv");
  hipLaunchKernelGGL(attn_bwd_q_kernel, dim3((T + DQ_Q - 1) / DQ_Q, B * H), dim3(256), 0, s, q, k, v, ld_qkv,
                     dout, ld_out, lse, delta, dq, H, T);
  GS_LAUNCH_CHECK("attn_bwd_q");
  return 0;
}

}  // namespace gs
