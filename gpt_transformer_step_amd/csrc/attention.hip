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
// Backward (one workgroup = 128 keys, 4 waves x 32 keys, looping over query
// tiles of 64): recompute S = Q K^T and P = exp(S - lse), dV^T += dO^T P,
// dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS; dS goes through LDS for
// dQ = dS K, which is accumulated in fp32 with atomics (dQ receives a
// contribution from every key block).

#include "common.h"
#include "kernels.h"

namespace gs {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int sw(int r) { return r & 7; }
// rows of 256 bytes (16 chunks of 16 B)
__device__ __forceinline__ int off256(int r, int c) { return r * 256 + ((c ^ sw(r)) << 4); }
// rows of 128 bytes (8 chunks of 16 B)
__device__ __forceinline__ int off128(int r, int c) { return r * 128 + ((c ^ sw(r)) << 4); }

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// transpose an 8x8 bf16 block held as 8 rows of 16 B: out[c] = column c
__device__ __forceinline__ void transpose8x8(const uint4* in, uint4* out) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int d = c >> 1;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = reinterpret_cast<const uint32_t*>(&in[2 * q])[d];
      const uint32_t b = reinterpret_cast<const uint32_t*>(&in[2 * q + 1])[d];
      w[q] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    out[c] = make_uint4(w[0], w[1], w[2], w[3]);
  }
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
    uint4 t[8];
    transpose8x8(L.v, t);
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4*>(svt + off128(eb * 8 + c, kb)) = t[c];
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
      // scale, mask, tile max
      float x[32];
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + kt * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
          const float val = (key <= myq && key < T) ? s[kt][e] * c : -INFINITY;
          x[kt * 16 + e] = val;
          tmax = fmaxf(tmax, val);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mnew = fmaxf(m, tmax);
      const float mref = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = exp2f(m - mref);
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        x[i] = exp2f(x[i] - mref);
        psum += x[i];
      }
      l = l * alpha + psum;
      m = mnew;
#pragma unroll
      for (int et = 0; et < 4; ++et)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[et][e] *= alpha;
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
constexpr int BKEYS = 128;  // keys per workgroup
constexpr int BQT = 64;     // queries per tile

// delta[b,h,t] = sum_e dout * out; also zero dq_acc. One wave per (token, head).
__global__ void attn_bwd_pre_kernel(const uint16_t* __restrict__ out, const uint16_t* __restrict__ dout,
                                    long long ld_out, float* __restrict__ delta, float* __restrict__ dq_acc,
                                    int H, int T, long long NH) {
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= NH) return;
  const long long n = w / H;
  const int h = (int)(w % H);
  const uint16_t* o = out + n * ld_out + h * 128;
  const uint16_t* d = dout + n * ld_out + h * 128;
  const uint32_t ow = reinterpret_cast<const uint32_t*>(o)[lane];
  const uint32_t dw = reinterpret_cast<const uint32_t*>(d)[lane];
  float s = lo_bf(ow) * lo_bf(dw) + hi_bf(ow) * hi_bf(dw);
  s = wave_sum(s);
  const long long b = n / T, t = n % T;
  if (lane == 0) delta[(b * H + h) * T + t] = s;
  float2* dq = reinterpret_cast<float2*>(dq_acc + n * (long long)H * 128 + h * 128);
  dq[lane] = make_float2(0.f, 0.f);
}

constexpr int B_QN = 0;                      // Q natural   [64][256 B]
constexpr int B_QT = B_QN + BQT * 256;       // Q^T         [128][128 B]
constexpr int B_DN = B_QT + 128 * 128;       // dO natural  [64][256 B]
constexpr int B_DT = B_DN + BQT * 256;       // dO^T        [128][128 B]
constexpr int B_DS = B_DT + 128 * 128;       // dS          [64 q][256 B = 128 keys]
constexpr int B_KT = B_DS + BQT * 256;       // K^T         [128 e][256 B = 128 keys]
constexpr int B_LSE = B_KT + 128 * 256;      // lse * log2e [64] fp32
constexpr int B_DEL = B_LSE + BQT * 4;       // delta       [64] fp32
constexpr int B_TOTAL = B_DEL + BQT * 4;

__global__ void __launch_bounds__(256, 1)
attn_bwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                long long ld, const uint16_t* __restrict__ dout, long long ld_out, const float* __restrict__ lse,
                const float* __restrict__ delta, float* __restrict__ dq_acc, uint16_t* __restrict__ dk,
                uint16_t* __restrict__ dv, long long ld_dkv, int H, int T) {
  __shared__ __attribute__((aligned(16))) char smem[B_TOTAL];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int nkb = (T + BKEYS - 1) / BKEYS;
  const int kb = blockIdx.x;  // key block; the early blocks (most query tiles) come first
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const long long rowbase = (long long)b * T;
  const int d = H * 128;
  const uint16_t* qh = q + rowbase * ld + h * 128;
  const uint16_t* kh = k + rowbase * ld + h * 128;
  const uint16_t* vh = v + rowbase * ld + h * 128;
  const uint16_t* doh = dout + rowbase * ld_out + h * 128;
  const float* lseh = lse + (long long)bh * T;
  const float* delh = delta + (long long)bh * T;
  const float scale = 0.08838834764831845f;
  const float c = scale * kLog2e;
  (void)nkb;

  const int k0 = kb * BKEYS;
  const int wk0 = k0 + wave * 32;
  const int mykey = wk0 + lr;  // this lane's key (column of S, P, dS)

  // K and V fragments of the wave's 32 keys (B operand: column = key)
  bf16x8_t fk[8], fv[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (mykey < T) {
      const uint4 a = ld16(kh + (long long)mykey * ld + ks * 16 + lh * 8);
      const uint4 bq = ld16(vh + (long long)mykey * ld + ks * 16 + lh * 8);
      fk[ks] = *reinterpret_cast<const bf16x8_t*>(&a);
      fv[ks] = *reinterpret_cast<const bf16x8_t*>(&bq);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { fk[ks][e] = 0; fv[ks][e] = 0; }
    }
  }
  // K^T of the whole key block in LDS (for dQ = dS K)
  {
    const int kbk = tid & 15, eb = tid >> 4;  // keys kbk*8.., features eb*8..
    uint4 blk[8], t8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = k0 + kbk * 8 + j;
      blk[j] = key < T ? ld16(kh + (long long)key * ld + eb * 8) : make_uint4(0, 0, 0, 0);
    }
    transpose8x8(blk, t8);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) *reinterpret_cast<uint4*>(smem + B_KT + off256(eb * 8 + cc, kbk)) = t8[cc];
  }

  f32x16_t dvt[4], dkt[4];
#pragma unroll
  for (int et = 0; et < 4; ++et)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dvt[et][e] = 0.f; dkt[et][e] = 0.f; }

  const int qt_first = k0 / BQT;
  const int nqt = (T + BQT - 1) / BQT;

  // loader: threads 0..127 an 8x8 block of Q, 128..255 of dO
  auto load_tile = [&](int qt, uint4* blk) {
    const int t = tid & 127;
    const int qb8 = t & 7, eb = t >> 3;  // queries qb8*8.., features eb*8..
    const uint16_t* base = (tid < 128) ? qh : doh;
    const long long ldx = (tid < 128) ? ld : ld_out;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int qq = qt * BQT + qb8 * 8 + j;
      blk[j] = qq < T ? ld16(base + (long long)qq * ldx + eb * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int qt, const uint4* blk) {
    const int t = tid & 127;
    const int qb8 = t & 7, eb = t >> 3;
    char* nat = smem + ((tid < 128) ? B_QN : B_DN);
    char* tr = smem + ((tid < 128) ? B_QT : B_DT);
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(nat + off256(qb8 * 8 + j, eb)) = blk[j];
    uint4 t8[8];
    transpose8x8(blk, t8);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) *reinterpret_cast<uint4*>(tr + off128(eb * 8 + cc, qb8)) = t8[cc];
    if (tid < BQT) {
      const int qq = qt * BQT + tid;
      reinterpret_cast<float*>(smem + B_LSE)[tid] = qq < T ? lseh[qq] * kLog2e : INFINITY;
      reinterpret_cast<float*>(smem + B_DEL)[tid] = qq < T ? delh[qq] : 0.f;
    }
  };

  uint4 pre[8];
  if (qt_first < nqt) {
    load_tile(qt_first, pre);
    store_tile(qt_first, pre);
  }
  __syncthreads();

  const float* slse = reinterpret_cast<const float*>(smem + B_LSE);
  const float* sdel = reinterpret_cast<const float*>(smem + B_DEL);

  for (int qt = qt_first; qt < nqt; ++qt) {
    const bool more = qt + 1 < nqt;
    if (more) load_tile(qt + 1, pre);
    const int q0 = qt * BQT;

    // S = Q K^T and dP = dO V^T for the two 32-query halves
    f32x16_t s[2], dp[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) { s[h2][e] = 0.f; dp[h2][e] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t aq = *reinterpret_cast<const bf16x8_t*>(smem + B_QN + off256(h2 * 32 + lr, ks * 2 + lh));
        const bf16x8_t ad = *reinterpret_cast<const bf16x8_t*>(smem + B_DN + off256(h2 * 32 + lr, ks * 2 + lh));
        s[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, fk[ks], s[h2], 0, 0, 0);
        dp[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, fv[ks], dp[h2], 0, 0, 0);
      }
    }
    // P and dS; element (h2, e) is query q0 + 32 h2 + 8 (e/4) + 4 lh + e%4, key mykey
    float p[32], ds[32];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ql = h2 * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
        const int qq = q0 + ql;
        float pv = exp2f(s[h2][e] * c - slse[ql]);
        pv = (mykey <= qq && mykey < T) ? pv : 0.f;
        p[h2 * 16 + e] = pv;
        ds[h2 * 16 + e] = pv * (dp[h2][e] - sdel[ql]);
      }
    // dV^T += dO^T P ; dK^T += Q^T dS  (k-steps of 16 queries, accumulator order)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8_t fp = pack_perm(p + (st >> 1) * 16, st & 1);
      const bf16x8_t fs = pack_perm(ds + (st >> 1) * 16, st & 1);
#pragma unroll
      for (int et = 0; et < 4; ++et) {
        const bf16x8_t ad = read_perm_frag(smem + B_DT, et * 32 + lr, st, lh);
        const bf16x8_t aq = read_perm_frag(smem + B_QT, et * 32 + lr, st, lh);
        dvt[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, fp, dvt[et], 0, 0, 0);
        dkt[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, fs, dkt[et], 0, 0, 0);
      }
    }
    // dS to LDS as [query][key] (keys of the whole block)
    {
      uint16_t* sds = reinterpret_cast<uint16_t*>(smem + B_DS);
      const int key_local = wave * 32 + lr;
      const int kc = key_local >> 3, kw = key_local & 7;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int ql = h2 * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
          sds[(off256(ql, kc) >> 1) + kw] = f2bf(ds[h2 * 16 + e]);
        }
    }
    __syncthreads();
    // dQ[q, e] += scale * sum_key dS[q, key] K[key, e]; wave owns features wave*32..+31
    {
      f32x16_t acc[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[h2][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(smem + B_DS + off256(h2 * 32 + lr, ks * 2 + lh));
          const bf16x8_t bk = *reinterpret_cast<const bf16x8_t*>(smem + B_KT + off256(wave * 32 + lr, ks * 2 + lh));
          acc[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bk, acc[h2], 0, 0, 0);
        }
      }
      // accumulator: column = feature wave*32 + lr, rows = queries 8g + 4lh + r
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int qq = q0 + h2 * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
          if (qq < T)
            unsafeAtomicAdd(dq_acc + (rowbase + qq) * d + h * 128 + wave * 32 + lr, acc[h2][e] * scale);
        }
    }
    __syncthreads();
    if (more) store_tile(qt + 1, pre);
    __syncthreads();
  }

  // dK = scale * dK^T^T, dV: lane owns key mykey, features et*32 + 8g + 4lh + r
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
                    float* dq_acc, uint16_t* dk, uint16_t* dv, long long ld_dkv, int B, int H, int T,
                    hipStream_t s) {
  if (B <= 0 || T <= 0) return 0;
  const long long NH = (long long)B * T * H;
  hipLaunchKernelGGL(attn_bwd_pre_kernel, dim3((unsigned)((NH + 3) / 4)), dim3(256), 0, s, out, dout, ld_out,
                     delta, dq_acc, H, T, NH);
  GS_LAUNCH_CHECK("attn_bwd_pre");
  dim3 grid((T + BKEYS - 1) / BKEYS, B * H);
  hipLaunchKernelGGL(attn_bwd_kernel, grid, dim3(256), 0, s, q, k, v, ld_qkv, dout, ld_out, lse, delta, dq_acc,
                     dk, dv, ld_dkv, H, T);
  GS_LAUNCH_CHECK("attn_bwd");
  return 0;
}

}  // namespace gs
