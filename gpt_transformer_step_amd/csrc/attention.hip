// Causal flash attention forward and backward, head width 128, on CDNA4
// matrix cores (v_mfma_f32_32x32x16_bf16).
//
// The model passage (dev.to "¿Cómo Entrenar Tu Propio ChatGPT por $50?",
// "1. Modelo GPT" and "5. Unificación Flash Attention") calls
// flash_attn_func(q, k, v, causal=True): y_t = sum_{j<=t} softmax_j(q_t.k_j /
// sqrt(128)) v_j, keeping row statistics (online softmax) instead of the
// T x T score matrix.
//
// Layout and data movement (gfx950):
//   * every LDS tile is a block of rows of 128 features (256 bytes) stored as
//     in HBM, filled by direct buffer->LDS loads (buffer_load_dwordx4 ... lds);
//     rows past the sequence end are clamped to a valid row (they are always
//     masked, so only finiteness matters);
//   * 16-byte chunks are XOR-swizzled by sigma(r) = 4 (r & 3) + ((r >> 2) & 3),
//     which keeps both access kinds free of bank conflicts: 16-byte fragment
//     reads of 16 consecutive rows, and transpose reads (ds_read_b64_tr_b16)
//     of 4 consecutive rows x 32 features;
//   * operands needed transposed (V^T, K^T, Q^T, dO^T) come straight from the
//     untransposed tiles through the transpose read, in the key order the
//     accumulators of P / dS use, so P and dS feed the next product directly
//     from registers.
// Forward: one workgroup = 128 queries (4 waves x 32) of one (batch, head).
//   Each wave computes S^T = K Q^T, so a lane owns one query (its partner
//   lane ^ 32 the other half of the keys): row max = one lane swap per tile,
//   row sum = none until the end.  O^T += V^T P^T with P rounded to bf16 and
//   the row sum l of the unrounded P (fp32), O = O / l at the end.  The
//   reference max moves only when a row max exceeds it by 2^8 (P <= 256), so
//   most tiles skip the O rescale.  K/V tiles of 64 keys, double buffered.
// Backward, two kernels and no atomics:
//   * dK/dV: one workgroup = 128 keys (4 waves x 32), two per CU, over
//     query tiles of 32 streamed through a 2-stage LDS ring: S = Q K^T, dP = dO V^T,
//     P = exp(S - lse), dS = P (dP - delta), dV^T += dO^T P, dK^T += Q^T dS;
//   * dQ (launched first): one workgroup = 128 queries over key tiles of 64,
//     shaped like the forward: S^T, dP^T recomputed, dQ^T += K^T dS^T; it
//     also computes delta = rowsum(dO O) of its queries and stores -delta for
//     the dK/dV kernel (whose dP accumulates onto it).
//   The dQ kernel recomputes two of the four products; in exchange dQ needs no
//   fp32 atomics and the result is deterministic.

#include "common.h"
#include "kernels.h"

namespace gs {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;                // log2 of the largest unnormalised P
constexpr float kScale = 0.08838834764831845f;  // 1 / sqrt(128)

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ int sigma(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// byte offset of 16-byte chunk c (features 8c .. 8c+7) of row r
__device__ __forceinline__ int toff(int r, int c) { return r * 256 + ((c ^ sigma(r)) << 4); }

__device__ __forceinline__ bf16x8_t frag16(const char* lds, int r, int c) {
  return *reinterpret_cast<const bf16x8_t*>(lds + toff(r, c));
}

__device__ __forceinline__ v4s_t tr_read(const char* lds, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)((const lds_char*)lds + byte_off));
}

// A-operand fragment of the transposed tile (MFMA rows = features et*32 ..
// et*32+31, k = 16 tile rows of step st in accumulator order: rows
// 16 st + 4 lh + 0..3, then 16 st + 8 + 4 lh + 0..3).  Transpose read
// semantics: within a 16-lane group, lane j gets element j % 4 of the 8 bytes
// loaded by lanes 4t + j/4 (t = 0..3).
__device__ __forceinline__ bf16x8_t frag_tr(const char* lds, int et, int st, int lane) {
  const int g = lane >> 4, m = lane & 15;
  const int i = et * 32 + 16 * (g & 1) + 4 * (m & 3);
  const int r = 16 * st + 4 * (g >> 1) + (m >> 2);
  const int sub = (i & 7) * 2;
  const v4s_t a = tr_read(lds, toff(r, i >> 3) + sub);
  const v4s_t b = tr_read(lds, toff(r + 8, i >> 3) + sub);
  bf16x8_t f;
  f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
  f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
  return f;
}

// pack accumulator values 8 s .. 8 s + 7 of x as bf16 (the B fragment of k-step s)
__device__ __forceinline__ bf16x8_t pack_perm(const float* x, int s) {
  bf16x8_t f;
  uint32_t* w = reinterpret_cast<uint32_t*>(&f);
  w[0] = pack_bf2(x[8 * s + 0], x[8 * s + 1]);
  w[1] = pack_bf2(x[8 * s + 2], x[8 * s + 3]);
  w[2] = pack_bf2(x[8 * s + 4], x[8 * s + 5]);
  w[3] = pack_bf2(x[8 * s + 6], x[8 * s + 7]);
  return f;
}

// An empty statement the compiler may not move or drop: placed in the body of
// a wave-uniform branch it keeps the branch, where the compiler would
// otherwise turn a cheap-looking body into selects executed on every pass.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// max of three floats in one instruction: the scores are finite or -inf, so
// the NaN quieting fmaxf adds in front of every operand is not needed
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Buffer resource (raw byte addressing, range num_bytes; gfx9 layout: base,
// base_hi | stride 0, num_records, format word) from wave-uniform values.
typedef int v4i_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i_t buf_rsrc(const void* base, long long num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int)min(num_bytes, (long long)0x7fffffff));
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// Direct buffer -> LDS loads of this kernel, written as instructions the
// compiler does not model: it would otherwise make every LDS read wait for
// every such load in flight (it cannot tell the ring's stages apart), which
// defeats loading several tiles ahead.  Ordering is the kernel's own: the
// loads into a stage are issued after the barrier that ends its last reads,
// and the barrier before its next reads follows an explicit vmcnt wait.
// They have no register results; "memory" keeps the compiler from moving LDS
// accesses across them.  M0 (the LDS base of the wave's write) is set here
// only; nothing compiled in this kernel reads M0.
__device__ __forceinline__ void dma16(v4i_t rsrc, int voffset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %0, 0 offen lds"
               :: "s"(rsrc), "v"(voffset), "s"(lds_base) : "memory");
}
__device__ __forceinline__ void dma4(v4i_t rsrc, int voffset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %1, %0, 0 offen lds"
               :: "s"(rsrc), "v"(voffset), "s"(lds_base) : "memory");
}

// Register operands loaded before a loop of direct loads: a use here makes
// the compiler wait for them now, in the prologue (otherwise it may sink the
// loads and wait for them inside the loop, where the counter also covers the
// direct loads of the next tile).
__device__ __forceinline__ void settle(const bf16x8_t& f) { asm volatile("" :: "v"(f)); }
__device__ __forceinline__ void settle(const float& f) { asm volatile("" :: "v"(f)); }

// Barrier after direct loads: the compiler does not see those loads, so the
// wait for them (and for any other load in flight) is explicit; it also tells
// the compiler that its own earlier loads have landed.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  __syncthreads();
  asm volatile("" ::: "memory");
}

// Linear block index in an order that keeps all blocks of one (sequence,
// head) on one XCD: the dispatcher deals workgroups x + gx y round robin to
// the 8 XCDs, so consecutive blocks would otherwise fetch the same K/V (or
// Q/dO) stream into 8 different L2s.  Each XCD instead walks a contiguous run
// of heads, one head's blocks after another, keeping the head's stream
// resident in its own L2.
__device__ __forceinline__ int xcd_block(int gx) {
  return xcd_remap(blockIdx.x + gx * blockIdx.y, gx * gridDim.y);
}

// RMS-norm + rotary backward of one 128-wide q or k head (the model's QK
// normalisation after the rotation), fused into the epilogue of the attention
// backward kernels.  acc holds the head's gradient in accumulator order: lane
// half lh holds features et*32 + 8*(e>>2) + 4*lh + (e&3) of element e of
// acc[et], the partner lane ^ 32 the other half.  With dy = scale * acc the
// gradient of the stored normed, rotated head y (bf16 row yrow) and r its
// inverse RMS: dx = r (dy - y mean(dy y)), then the inverse rotation of the
// pairs (i, i + 64) at position t (cos table [T][64], then sin [T][64]); the
// result goes out as bf16.  Features i and i + 64 sit in acc[et] and
// acc[et + 2] of the same lane, so the rotation needs no exchange.
// max |value| of the two bf16 values of a stored word pair
__device__ __forceinline__ float absmax_w(uint2 w) {
  return fmaxf(fmaxf(fabsf(lo_bf(w.x)), fabsf(hi_bf(w.x))), fmaxf(fabsf(lo_bf(w.y)), fabsf(hi_bf(w.y))));
}

// One wave's max |stored value| into amax[slot] (fp8 scale partials; no-op
// without amax).  Every lane of the wave calls it.
__device__ __forceinline__ void store_wave_amax(float* amax, long long slot, float m) {
  if (!amax) return;
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) amax[slot] = m;
}

// Returns the max |stored value| of the lane.
__device__ __forceinline__ float qknorm_rope_bwd_store(const f32x16_t* acc, float scale, const uint16_t* yrow, float r,
                                                      const float* cs, int T, int t, int lh, uint16_t* out) {
  uint2 yw[4][4];
  float dot = 0.f;
#pragma unroll
  for (int et = 0; et < 4; ++et)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      yw[et][g] = *reinterpret_cast<const uint2*>(yrow + et * 32 + 8 * g + 4 * lh);
      dot += acc[et][4 * g] * lo_bf(yw[et][g].x) + acc[et][4 * g + 1] * hi_bf(yw[et][g].x) +
             acc[et][4 * g + 2] * lo_bf(yw[et][g].y) + acc[et][4 * g + 3] * hi_bf(yw[et][g].y);
    }
  dot += __shfl_xor(dot, 32, 64);
  const float mean = dot * scale * (1.f / 128.f);
  float amx = 0.f;
  const float* cr = cs + t * 64;
  const float* sr = cs + (long long)T * 64 + t * 64;
#pragma unroll
  for (int et = 0; et < 2; ++et)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int i = et * 32 + 8 * g + 4 * lh;
      const float4 c = *reinterpret_cast<const float4*>(cr + i);
      const float4 sn = *reinterpret_cast<const float4*>(sr + i);
      const float y1[4] = {lo_bf(yw[et][g].x), hi_bf(yw[et][g].x), lo_bf(yw[et][g].y), hi_bf(yw[et][g].y)};
      const float y2[4] = {lo_bf(yw[et + 2][g].x), hi_bf(yw[et + 2][g].x), lo_bf(yw[et + 2][g].y),
                           hi_bf(yw[et + 2][g].y)};
      const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
      float o1[4], o2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float d1 = r * (acc[et][4 * g + u] * scale - y1[u] * mean);
        const float d2 = r * (acc[et + 2][4 * g + u] * scale - y2[u] * mean);
        o1[u] = d1 * cc[u] + d2 * ss[u];
        o2[u] = -d1 * ss[u] + d2 * cc[u];
      }
      const uint2 w1 = make_uint2(pack_bf2(o1[0], o1[1]), pack_bf2(o1[2], o1[3]));
      const uint2 w2 = make_uint2(pack_bf2(o2[0], o2[1]), pack_bf2(o2[2], o2[3]));
      *reinterpret_cast<uint2*>(out + i) = w1;
      *reinterpret_cast<uint2*>(out + i + 64) = w2;
      amx = fmaxf(amx, fmaxf(absmax_w(w1), absmax_w(w2)));
    }
  return amx;
}

// Copy of ROWS rows of 128 features (row r0 + r clamped to T - 1) of a bf16
// matrix whose row 0 is byte 0 of rsrc into a swizzled tile, by NT threads:
// round i, wave w, lane l fills 16-byte slot NT i + 64 w + l.  Offsets
// (row * ld + chunk) * 2 fit 32 bits (T <= 16384, ld < 2^16).
template <int ROWS, int NT>
__device__ __forceinline__ void tile_dma(v4i_t rsrc, int ld, int r0, int T, char* lds, int tid) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
  for (int i = 0; i < ROWS * 16 / NT; ++i) {
    const int slot = tid + NT * i;
    const int r = slot >> 4, c = (slot & 15) ^ sigma(r);
    const int row = min(r0 + r, T - 1);
    dma16(rsrc, (row * ld + c * 8) * 2, lds_addr(lds + (NT * i + 64 * wave) * 16));
  }
}

// ============================================================================
// forward
// ============================================================================
constexpr int FQ = 128;                // queries per workgroup
constexpr int FK = 64;                 // keys per tile
constexpr int F_STAGE = 2 * FK * 256;  // K tile + V tile

// GEN = false compiles the plain case (every head its own key/value head, no
// window) without the index arithmetic of the general one.
template <bool GEN>
__global__ void __launch_bounds__(256, 2)
attn_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                long long ld, uint16_t* __restrict__ out, long long ld_out, float* __restrict__ lse, int H, int Hkv,
                int T, int window_arg, int lse_log2, float* __restrict__ amax) {
  __shared__ __attribute__((aligned(16))) char smem[2 * F_STAGE];
  const int window = GEN ? window_arg : -1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int nqb = (T + FQ - 1) / FQ;
  const int bx = xcd_block(gridDim.x), bhq = bx / gridDim.x;
  const int qb = nqb - 1 - (bx - bhq * gridDim.x);  // longest rows first
  const int bh = bhq, b = bh / H, h = bh % H;
  const int hk = GEN ? h / (H / Hkv) : h;  // key/value head of this query head
  const long long rowbase = (long long)b * T;
  const uint16_t* qh = q + rowbase * ld + h * 128;
  const uint16_t* kh = k + rowbase * ld + hk * 128;
  const uint16_t* vh = v + rowbase * ld + hk * 128;

  const int q0 = qb * FQ;
  const int wq0 = q0 + wave * 32;   // first query of this wave
  const int myq = wq0 + lr;         // this lane's query
  const float c = kScale * kLog2e;  // scores in log2 units

  // Q fragments (B operand: column = query, 8 features per k-step)
  bf16x8_t fq[8];
  {
    const int qrow = min(myq, T - 1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 w = ld16(qh + (long long)qrow * ld + ks * 16 + lh * 8);
      fq[ks] = *reinterpret_cast<const bf16x8_t*>(&w);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) settle(fq[ks]);
  }

  f32x16_t o[4];
#pragma unroll
  for (int et = 0; et < 4; ++et)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[et][e] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int last_key = min(T - 1, q0 + FQ - 1);
  const int ntiles = last_key / FK + 1;
  const int j0 = window >= 0 ? max(0, q0 - window) / FK : 0;  // first key tile any query of the block sees

  const v4i_t rk = buf_rsrc(kh, (long long)T * ld * 2), rv = buf_rsrc(vh, (long long)T * ld * 2);
  tile_dma<FK, 256>(rk, (int)ld, j0 * FK, T, smem, tid);
  tile_dma<FK, 256>(rv, (int)ld, j0 * FK, T, smem + FK * 256, tid);
  dma_barrier();

  for (int j = j0; j < ntiles; ++j) {
    const char* sk = smem + ((j - j0) & 1) * F_STAGE;
    const char* sv = sk + FK * 256;
    if (j + 1 < ntiles) {  // block-uniform; the other stage was last read before the previous barrier
      char* nk = smem + ((j + 1 - j0) & 1) * F_STAGE;
      tile_dma<FK, 256>(rk, (int)ld, (j + 1) * FK, T, nk, tid);
      tile_dma<FK, 256>(rv, (int)ld, (j + 1) * FK, T, nk + FK * 256, tid);
    }
    const int key0 = j * FK;
    // wave-uniform: some key of the tile is visible to some query of the wave
    if (key0 <= wq0 + 31 && (window < 0 || key0 + FK - 1 >= wq0 - window)) {
      // S^T over the 64 keys: the two 32-key halves' MFMAs alternate, with
      // each k-step's K fragments read one k-step ahead
      f32x16_t s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
      bf16x8_t fk[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) fk[0][kt] = frag16(sk, kt * 32 + lr, lh);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (ks + 1 < 8) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) fk[(ks + 1) & 1][kt] = frag16(sk, kt * 32 + lr, (ks + 1) * 2 + lh);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[ks & 1][kt], fq[ks], s[kt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool diag = (key0 + FK - 1 > wq0) || (key0 + FK > T) || (window >= 0 && key0 < wq0 + 31 - window);
      // raw scores; the max is taken on raw scores (c > 0) and the scale is
      // folded into the exponent: p = exp2(s c - m)
      float x[32];
      if (diag) {
        keep_branch();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = key0 + kt * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
            const bool vis = key <= myq && key < T && (window < 0 || key >= myq - window);
            x[kt * 16 + e] = vis ? s[kt][e] : -INFINITY;
          }
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) x[kt * 16 + e] = s[kt][e];
      }
      // row max as four independent chains of 8 (dependency depth 6, not 16)
      float t4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        t4[j] = max3(max3(max3(x[8 * j], x[8 * j + 1], x[8 * j + 2]), x[8 * j + 3], x[8 * j + 4]), x[8 * j + 5],
                     fmaxf(x[8 * j + 6], x[8 * j + 7]));
      float tmax = fmaxf(max3(t4[0], t4[1], t4[2]), t4[3]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * c;
      const bool need = tmax > m + kRescale;
      if (__any(need)) {
        // lanes that keep their max scale by 1; with a window a lane may still
        // be at m = -inf here while another lane of the wave sees its first key
        const float mn = need ? tmax : m;
        const float alpha = need ? __builtin_amdgcn_exp2f(m - mn) : 1.f;
        l *= alpha;
        m = mn;
#pragma unroll
        for (int et = 0; et < 4; ++et)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[et][e] *= alpha;
      }
      // a row that has seen no visible key yet keeps m = -inf; its p are 0
      const float msafe = m == -INFINITY ? 0.f : m;
      float ps4[4] = {0.f, 0.f, 0.f, 0.f};  // four independent partial sums
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c, -msafe));
        ps4[i & 3] += x[i];
      }
      l += (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
      // O^T += V^T P^T over the 64 keys (4 k-steps of 16)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8_t fp = pack_perm(x, st);
#pragma unroll
        for (int et = 0; et < 4; ++et)
          o[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr(sv, et, st, lane), fp, o[et], 0, 0, 0);
      }
    }
    dma_barrier();  // the next tile has landed; every wave is done with this one
  }

  l += __shfl_xor(l, 32, 64);
  float amx = 0.f;  // max |stored value| of the lane (fp8 scale partials)
  if (myq < T) {
    const float inv = 1.f / l;
    uint16_t* orow = out + (rowbase + myq) * ld_out + h * 128;
#pragma unroll
    for (int et = 0; et < 4; ++et)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = et * 32 + 8 * g + 4 * lh;
        const uint2 w = make_uint2(pack_bf2(o[et][4 * g] * inv, o[et][4 * g + 1] * inv),
                                   pack_bf2(o[et][4 * g + 2] * inv, o[et][4 * g + 3] * inv));
        *reinterpret_cast<uint2*>(orow + e) = w;
        amx = fmaxf(amx, absmax_w(w));
      }
    // lse_log2: in log2 units (the backward kernels' exponent), else natural
    if (lh == 0) lse[(long long)bh * T + myq] = lse_log2 ? m + __log2f(l) : m * kLn2 + logf(l);
  }
  store_wave_amax(amax, ((long long)blockIdx.x + (long long)gridDim.x * blockIdx.y) * 4 + wave, amx);
}

// ============================================================================
// backward
// ============================================================================
// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
constexpr int KV_Q = 32;  // queries per tile

// ---------------------------------------------------------------------------
// One workgroup = 128 keys (4 waves x 32) of one (batch, key/value head),
// two workgroups per CU; Q / dO tiles of 32 queries and their softmax
// statistics stream through a ring of K8_NS LDS stages filled by direct
// buffer -> LDS loads issued K8_NS - 1 tiles ahead.  Two independent
// workgroups on a CU (one wave of each per SIMD) drift apart between their
// barriers, so one's exponentials and LDS reads run under the other's MFMAs;
// with one workgroup of 256 keys and a 4-stage ring every wave of a SIMD sat
// in the same phase (18.6 against 22.7 ms per d20 step).  The end-of-tile
// barrier waits for the next tile's loads (vmcnt).  Buffer loads take a
// scalar base and one 32-bit offset per thread, which keeps the streaming
// loads' addresses out of the (fully used) vector register budget.
// ---------------------------------------------------------------------------
constexpr int K8_KEYS = 128;
constexpr int K8_NT = 256;
// LDS: K of the block [128][256 B] and K8_NS ring stages, each its own
// __shared__ array of Q [32][256 B], dO [32][256 B], lse [32] and -delta [32].
// Separate arrays carry separate alias scopes, so the compiler can tell that
// an LDS read of one stage does not depend on the direct loads in flight into
// another (with a single array it waits for all of them before every read).
// The loop is unrolled by K8_NS so that each copy names its stages statically.
constexpr int K8_NS = 2;
constexpr int K8_QN = 0, K8_DN = KV_Q * 256, K8_ST = 2 * KV_Q * 256;
constexpr int K8_STAGE = K8_ST + 2 * KV_Q * 4;
constexpr int K8_TOTAL = K8_KEYS * 256 + K8_NS * K8_STAGE;
constexpr int K8_LOADS = 2 * (KV_Q * 16 / K8_NT) + 1;  // direct loads per thread per query tile
// s_waitcnt immediate (gfx9 encoding): vmcnt = loads of the K8_NS - 2 tiles
// issued after the next one (none with two stages); expcnt and lgkmcnt not
// waited for
constexpr int K8_VMCNT = K8_LOADS * (K8_NS - 2);
constexpr int K8_WAIT = (K8_VMCNT & 15) | ((K8_VMCNT >> 4) << 14) | (7 << 4) | (15 << 8);
static_assert(K8_TOTAL <= 160 * 1024, "LDS budget");
static_assert(K8_VMCNT < 64, "vmcnt range");

// FUSE: dK leaves through the QK-norm + rotary backward (rk: inverse RMS of
// each key head [N, Hkv]; cs: rotary table), else as the raw gradient.
template <bool GEN, bool FUSE>
__global__ void __launch_bounds__(K8_NT, 2)
attn_bwd_kv8_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                    long long ld, const uint16_t* __restrict__ dout, long long ld_out, const float* __restrict__ lse,
                    const float* __restrict__ delta, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                    long long ld_dkv, int H, int Hkv, int T, int window_arg, const float* __restrict__ rk,
                    const float* __restrict__ cs, float* __restrict__ amax) {
  static_assert(K8_NS == 2, "one __shared__ array per stage below");
  __shared__ __attribute__((aligned(16))) char s_k[K8_KEYS * 256];
  __shared__ __attribute__((aligned(16))) char s_st0[K8_STAGE];
  __shared__ __attribute__((aligned(16))) char s_st1[K8_STAGE];
  auto stage = [&](int j) -> char* { return j == 0 ? s_st0 : s_st1; };
  const int window = GEN ? window_arg : -1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int bx = xcd_block(gridDim.x), bhk = bx / gridDim.x;
  const int kb = bx - bhk * gridDim.x;
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int G = GEN ? H / Hkv : 1;
  const long long rowbase = (long long)b * T;
  const uint16_t* kh = k + rowbase * ld + hk * 128;
  const uint16_t* vh = v + rowbase * ld + hk * 128;
  const float c = kScale * kLog2e;

  const int k0 = kb * K8_KEYS;
  const int wk0 = k0 + wave * 32;
  const int mykey = wk0 + lr;

  f32x16_t dvt[4], dkt[4];
#pragma unroll
  for (int et = 0; et < 4; ++et)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dvt[et][e] = 0.f; dkt[et][e] = 0.f; }

  const int nqt = (T + KV_Q - 1) / KV_Q;
  const int qt_first = k0 / KV_Q;
  const int qt_end = window >= 0 ? min(nqt, (k0 + K8_KEYS - 1 + window) / KV_Q + 1) : nqt;
  const int nq = max(0, qt_end - qt_first);
  const int n_it = G * nq;  // (query head, query tile) pairs; block-uniform

  auto hq_of = [&](int it) { return GEN ? hk * G + it / nq : hk; };
  // query tiles from the last one down: every workgroup of a (sequence, head)
  // starts on the same tile, so blocks dispatched together read each Q / dO
  // tile at about the same time (one L2 fill serves them all); walking up
  // from its own diagonal, block kb would reach tile t at a different time
  // from every other block
  auto qt_of = [&](int it) { return GEN ? qt_end - 1 - it % nq : qt_end - 1 - it; };
  // the K8_LOADS direct loads of tile it (clamped to the last tile) into
  // stage st: Q and dO (two 16-byte chunks per thread each) and the
  // statistics (one per thread of lanes 0 .. PER - 1, below)
  auto issue = [&](int it, int st) {
    it = min(it, n_it - 1);
    const int hq = hq_of(it), q0 = qt_of(it) * KV_Q;
    char* so = stage(st);
    // an opaque thread index: the load offsets are recomputed per tile
    // rather than held across the loop
    int tid_o = tid;
    asm volatile("" : "+v"(tid_o));
    tile_dma<KV_Q, K8_NT>(buf_rsrc(q + rowbase * ld + hq * 128, (long long)T * ld * 2), (int)ld, q0, T, so + K8_QN,
                          tid_o);
    tile_dma<KV_Q, K8_NT>(buf_rsrc(dout + rowbase * ld_out + hq * 128, (long long)T * ld_out * 2), (int)ld_out, q0, T,
                          so + K8_DN, tid_o);
    // statistics: the first half of the waves load lse, the second -delta,
    // PER values each (lanes 0 .. PER - 1)
    constexpr int NWV = K8_NT / 64, PER = 2 * KV_Q / NWV;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const float* src = (wu < NWV / 2 ? lse : delta) + ((long long)b * H + hq) * T;
    const int qq = min(q0 + PER * (wu % (NWV / 2)) + (lane % PER), T - 1);
    const v4i_t rs = buf_rsrc(src, (long long)T * 4);
    if (lane < PER) dma4(rs, qq * 4, lds_addr(so + K8_ST + 4 * PER * wu));
  };

  if (n_it > 0) {
    tile_dma<K8_KEYS, K8_NT>(buf_rsrc(kh, (long long)T * ld * 2), (int)ld, k0, T, s_k, tid);
#pragma unroll
    for (int j = 0; j < K8_NS - 1; ++j) issue(j, j);
    // V fragments of the wave's keys in registers (B operand of dP = dO V^T)
    bf16x8_t fv[8];
    {
      const int vrow = min(mykey, T - 1);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint4 a = ld16(vh + (long long)vrow * ld + ks * 16 + lh * 8);
        fv[ks] = *reinterpret_cast<const bf16x8_t*>(&a);
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) settle(fv[ks]);
    }
    // everything of the prologue has landed (K, the first tiles, V)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // The lane's LDS byte offsets inside a tile, all below 2^16, two per
    // register, computed once: o16[k] the fragment reads of row lr at k-steps
    // 2k and 2k+1; otr[et] the two transpose reads of frag_tr(., et, 0, .)
    // (k-step s2 adds 16 rows, 4096 bytes).  Opaque to the compiler, so it
    // keeps these 8 registers instead of recomputing some 90 offset
    // instructions per tile (all 16 offsets unpacked do not fit beside the
    // accumulators).
    uint32_t o16[4], otr[4];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) o16[k2] = toff(lr, 4 * k2 + lh) | (toff(lr, 4 * k2 + 2 + lh) << 16);
    {
      const int g = lane >> 4, m = lane & 15;
      const int r = 4 * (g >> 1) + (m >> 2);
#pragma unroll
      for (int et = 0; et < 4; ++et) {
        const int i = et * 32 + 16 * (g & 1) + 4 * (m & 3);
        const int sub = (i & 7) * 2;
        otr[et] = (toff(r, i >> 3) + sub) | ((toff(r + 8, i >> 3) + sub) << 16);
      }
    }
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) asm volatile("" : "+v"(o16[k2]), "+v"(otr[k2]));
    const char* sk_w = s_k + __builtin_amdgcn_readfirstlane(wave) * 32 * 256;  // the wave's 32 keys
    auto off16 = [&](int ks) -> int {
      const uint32_t w = o16[ks >> 1];
      return (ks & 1) ? (int)(w >> 16) : (int)(w & 0xffffu);
    };
    auto frag_o = [&](const char* base, int off) -> bf16x8_t { return *reinterpret_cast<const bf16x8_t*>(base + off); };
    auto frag_tr_o = [&](const char* base, int et, int s2) -> bf16x8_t {
      const uint32_t w = otr[et];
      const v4s_t a = tr_read(base, (int)(w & 0xffffu) + 4096 * s2);
      const v4s_t b = tr_read(base, (int)(w >> 16) + 4096 * s2);
      bf16x8_t f;
      f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
      f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
      return f;
    };

    for (int it0 = 0; it0 < n_it; it0 += K8_NS)
#pragma unroll
    for (int cur = 0; cur < K8_NS; ++cur) {
      const int it = it0 + cur;
      if (it >= n_it) break;  // block-uniform
      const char* st = stage(cur);
      // tile it + K8_NS - 1 into the stage read during tile it - 1
      issue(it + K8_NS - 1, (cur + K8_NS - 1) % K8_NS);
      const int q0 = qt_of(it) * KV_Q;
      // wave-uniform: some query of the tile sees some key of the wave
      if (q0 + KV_Q - 1 >= wk0 && (window < 0 || q0 <= wk0 + 31 + window)) {
        // the scores first, then dP = dO V^T: P = exp2(S c - lse) needs only
        // the former and runs under the latter (same straight-line block)
        // dP accumulates onto -delta (stored negated by the dQ kernel), so it
        // leaves the products as dP - delta
        const float* slse = reinterpret_cast<const float*>(st + K8_ST);
        const float* sndel = slse + KV_Q;
        f32x16_t sacc, dpacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) { sacc[e] = 0.f; dpacc[e] = sndel[8 * (e >> 2) + 4 * lh + (e & 3)]; }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_o(st + K8_QN, off16(ks)), frag_o(sk_w, off16(ks)), sacc,
                                                         0, 0, 0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_o(st + K8_DN, off16(ks)), fv[ks], dpacc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int ql = 8 * (e >> 2) + 4 * lh + (e & 3);
          const float l2 = FUSE ? slse[ql] : slse[ql] * kLog2e;  // FUSE: lse stored in log2 units
          sacc[e] = __builtin_amdgcn_exp2f(sacc[e] * c - l2);  // P, in place of S
        }
        // rows past the sequence end carry the last row's statistics: masked
        const bool diag = (q0 < wk0 + 31) || (q0 + KV_Q > T) || (wk0 + 32 > T) ||
                          (window >= 0 && q0 + KV_Q - 1 > wk0 + window);
        if (diag) {  // wave-uniform: the visibility test only on tiles that need it
          keep_branch();
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int ql = 8 * (e >> 2) + 4 * lh + (e & 3);
            const bool vis =
                mykey <= q0 + ql && mykey < T && q0 + ql < T && (window < 0 || mykey >= q0 + ql - window);
            sacc[e] = __int_as_float(__float_as_int(sacc[e]) & -(int)vis);
          }
        }
        // P and dS = P (dP - delta) of the tile as bf16 B fragments
        bf16x8_t fp[2], fs[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          uint32_t* wp = reinterpret_cast<uint32_t*>(&fp[s2]);
          uint32_t* wd = reinterpret_cast<uint32_t*>(&fs[s2]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e0 = 8 * s2 + 2 * i, e1 = e0 + 1;
            wp[i] = pack_bf2(sacc[e0], sacc[e1]);
            wd[i] = pack_bf2(sacc[e0] * dpacc[e0], sacc[e1] * dpacc[e1]);
          }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int et = 0; et < 4; ++et) {
            dvt[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr_o(st + K8_DN, et, s2), fp[s2], dvt[et], 0, 0, 0);
            dkt[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr_o(st + K8_QN, et, s2), fs[s2], dkt[et], 0, 0, 0);
          }
      }
      // the next tile has landed (only the K8_NS - 2 tiles behind it may be in
      // flight) and every wave is done with this stage
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(K8_WAIT);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    // drain the trailing (re-issued) loads before the workgroup ends
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  }

  float amx = 0.f;  // max |stored dK, dV value| of the lane (fp8 scale partials)
  if (mykey < T) {
    uint16_t* dkr = dk + (rowbase + mykey) * ld_dkv + hk * 128;
    uint16_t* dvr = dv + (rowbase + mykey) * ld_dkv + hk * 128;
#pragma unroll
    for (int et = 0; et < 4; ++et)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = et * 32 + 8 * g + 4 * lh;
        if constexpr (!FUSE) {
          const uint2 w = make_uint2(pack_bf2(dkt[et][4 * g] * kScale, dkt[et][4 * g + 1] * kScale),
                                     pack_bf2(dkt[et][4 * g + 2] * kScale, dkt[et][4 * g + 3] * kScale));
          *reinterpret_cast<uint2*>(dkr + e) = w;
          amx = fmaxf(amx, absmax_w(w));
        }
        const uint2 w = make_uint2(pack_bf2(dvt[et][4 * g], dvt[et][4 * g + 1]),
                                   pack_bf2(dvt[et][4 * g + 2], dvt[et][4 * g + 3]));
        *reinterpret_cast<uint2*>(dvr + e) = w;
        amx = fmaxf(amx, absmax_w(w));
      }
    if constexpr (FUSE)
      amx = fmaxf(amx, qknorm_rope_bwd_store(dkt, kScale, kh + (long long)mykey * ld, rk[(rowbase + mykey) * Hkv + hk],
                                             cs, T, mykey, lh, dkr));
  }
  store_wave_amax(amax, ((long long)blockIdx.x + (long long)gridDim.x * blockIdx.y) * (K8_NT / 64) + wave, amx);
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
// (64 queries and 32-key tiles, four workgroups per CU, needed 276 registers,
// one wave per SIMD: dQ 14.3 -> 22.9 ms per d20 step)
constexpr int DQ_Q = 128;                  // queries per workgroup (32 per wave)
constexpr int DQ_NT = DQ_Q * 2;            // threads
constexpr int DQ_K = 64;                   // keys per tile
constexpr int DQ_KT = DQ_K / 32;           // 32-key blocks per tile
constexpr int DQ_STAGE = 2 * DQ_K * 256;  // K tile + V tile

// FUSE: dQ leaves through the QK-norm + rotary backward as bf16 into dq_bf
// (row stride ld_dq; rq: inverse RMS of each query head [N, H]; cs: rotary
// table), else as the raw fp32 gradient into dq_out (row stride 128 H).
template <bool GEN, bool FUSE>
__global__ void __launch_bounds__(DQ_NT, 512 / DQ_NT)
attn_bwd_q_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                  long long ld, const uint16_t* __restrict__ out, const uint16_t* __restrict__ dout, long long ld_out,
                  const float* __restrict__ lse, float* __restrict__ delta, float* __restrict__ dq_out, int H,
                  int Hkv, int T, int window_arg, uint16_t* __restrict__ dq_bf, long long ld_dq,
                  const float* __restrict__ rq, const float* __restrict__ cs, float* __restrict__ amax) {
  __shared__ __attribute__((aligned(16))) char smem[2 * DQ_STAGE];
  const int window = GEN ? window_arg : -1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lh = lane >> 5;
  const int nqb = (T + DQ_Q - 1) / DQ_Q;
  const int bx = xcd_block(gridDim.x), bhq = bx / gridDim.x;
  const int qb = nqb - 1 - (bx - bhq * gridDim.x);  // longest rows first
  const int bh = bhq, b = bh / H, h = bh % H;
  const int hk = GEN ? h / (H / Hkv) : h;
  const long long rowbase = (long long)b * T;
  const int d = H * 128;
  const uint16_t* qh = q + rowbase * ld + h * 128;
  const uint16_t* kh = k + rowbase * ld + hk * 128;
  const uint16_t* vh = v + rowbase * ld + hk * 128;
  const uint16_t* doh = dout + rowbase * ld_out + h * 128;
  const float c = kScale * kLog2e;

  const int q0 = qb * DQ_Q;
  const int wq0 = q0 + wave * 32;
  const int myq = wq0 + lr;
  bf16x8_t fq[8], fd[8];
  uint4 ow8[8];  // the same features of O (for delta), loaded in the same batch
  {
    const int qrow = min(myq, T - 1);
    const uint16_t* oh = out + rowbase * ld_out + h * 128;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 a = ld16(qh + (long long)qrow * ld + ks * 16 + lh * 8);
      const uint4 bq = ld16(doh + (long long)qrow * ld_out + ks * 16 + lh * 8);
      ow8[ks] = ld16(oh + (long long)qrow * ld_out + ks * 16 + lh * 8);
      fq[ks] = *reinterpret_cast<const bf16x8_t*>(&a);
      fd[ks] = *reinterpret_cast<const bf16x8_t*>(&bq);
    }
  }
  // FUSE: lse stored in log2 units by the forward
  const float lse2 = myq < T ? (FUSE ? lse[(long long)bh * T + myq] : lse[(long long)bh * T + myq] * kLog2e) : INFINITY;
  // delta = rowsum(dO * O) of this lane's query: the lane holds half of the
  // dO row (the fragments above), its partner lane ^ 32 the other half; the
  // dK/dV kernel, launched after this one, reads the stored values (negated)
  float del;
  {
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 ow = ow8[ks];
      const uint32_t* dw = reinterpret_cast<const uint32_t*>(&fd[ks]);
      part += lo_bf(ow.x) * lo_bf(dw[0]) + hi_bf(ow.x) * hi_bf(dw[0]) + lo_bf(ow.y) * lo_bf(dw[1]) +
              hi_bf(ow.y) * hi_bf(dw[1]) + lo_bf(ow.z) * lo_bf(dw[2]) + hi_bf(ow.z) * hi_bf(dw[2]) +
              lo_bf(ow.w) * lo_bf(dw[3]) + hi_bf(ow.w) * hi_bf(dw[3]);
    }
    part += __shfl_xor(part, 32, 64);
    del = myq < T ? part : 0.f;
    if (lh == 0 && myq < T) delta[(long long)bh * T + myq] = -part;  // negated: the dK/dV kernel's dP starts there
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    settle(fq[ks]);
    settle(fd[ks]);
  }
  settle(lse2);
  settle(del);

  f32x16_t dqt[4];
#pragma unroll
  for (int et = 0; et < 4; ++et)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqt[et][e] = 0.f;

  const int last_key = min(T - 1, q0 + DQ_Q - 1);
  const int ntiles = last_key / DQ_K + 1;
  const int j0 = window >= 0 ? max(0, q0 - window) / DQ_K : 0;
  const v4i_t rk = buf_rsrc(kh, (long long)T * ld * 2), rv = buf_rsrc(vh, (long long)T * ld * 2);
  tile_dma<DQ_K, DQ_NT>(rk, (int)ld, j0 * DQ_K, T, smem, tid);
  tile_dma<DQ_K, DQ_NT>(rv, (int)ld, j0 * DQ_K, T, smem + DQ_K * 256, tid);
  dma_barrier();

  for (int j = j0; j < ntiles; ++j) {
    const char* sk = smem + ((j - j0) & 1) * DQ_STAGE;
    const char* sv = sk + DQ_K * 256;
    if (j + 1 < ntiles) {
      char* nk = smem + ((j + 1 - j0) & 1) * DQ_STAGE;
      tile_dma<DQ_K, DQ_NT>(rk, (int)ld, (j + 1) * DQ_K, T, nk, tid);
      tile_dma<DQ_K, DQ_NT>(rv, (int)ld, (j + 1) * DQ_K, T, nk + DQ_K * 256, tid);
    }
    const int key0 = j * DQ_K;
    if (key0 <= wq0 + 31 && (window < 0 || key0 + DQ_K - 1 >= wq0 - window)) {  // wave-uniform
      // the scores first, then dP = dO V^T, as one run of 16 k-steps (K
      // fragments, then V) whose fragments are read one k-step ahead of the
      // MFMAs that use them (read next to their use, every MFMA waited for
      // its LDS read); the exponentials of the scores run between the dP
      // MFMAs, four per k-step
      f32x16_t st2[DQ_KT], dpt[DQ_KT];
#pragma unroll
      for (int kt = 0; kt < DQ_KT; ++kt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) { st2[kt][e] = 0.f; dpt[kt][e] = 0.f; }
      }
      float ds[DQ_KT * 16];
      bf16x8_t fkv[2][DQ_KT];
#pragma unroll
      for (int kt = 0; kt < DQ_KT; ++kt) fkv[0][kt] = frag16(sk, kt * 32 + lr, lh);
#pragma unroll
      for (int i = 0; i < 16; ++i) {  // i < 8: scores, k-step i; i >= 8: dP, k-step i - 8
        if (i + 1 < 16) {
#pragma unroll
          for (int kt = 0; kt < DQ_KT; ++kt)
            fkv[(i + 1) & 1][kt] = frag16(i + 1 < 8 ? sk : sv, kt * 32 + lr, ((i + 1) & 7) * 2 + lh);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt = 0; kt < DQ_KT; ++kt) {
          if (i < 8)
            st2[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fkv[i & 1][kt], fq[i], st2[kt], 0, 0, 0);
          else
            dpt[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fkv[i & 1][kt], fd[i - 8], dpt[kt], 0, 0, 0);
        }
        if (i >= 8) {
#pragma unroll
          for (int u = 0; u < DQ_KT * 2; ++u) {
            const int x = (i - 8) * DQ_KT * 2 + u;
            ds[x] = __builtin_amdgcn_exp2f(st2[x >> 4][x & 15] * c - lse2);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool diag = (key0 + DQ_K - 1 > wq0) || (key0 + DQ_K > T) || (window >= 0 && key0 < wq0 + 31 - window);
      if (diag) {  // wave-uniform: the visibility test only on tiles that need it
        keep_branch();
#pragma unroll
        for (int kt = 0; kt < DQ_KT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = key0 + kt * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
            const bool vis = key <= myq && key < T && (window < 0 || key >= myq - window);
            ds[kt * 16 + e] = vis ? ds[kt * 16 + e] : 0.f;
          }
      }
#pragma unroll
      for (int kt = 0; kt < DQ_KT; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) ds[kt * 16 + e] *= dpt[kt][e] - del;
#pragma unroll
      for (int s4 = 0; s4 < 2 * DQ_KT; ++s4) {
        const bf16x8_t fs = pack_perm(ds, s4);
#pragma unroll
        for (int et = 0; et < 4; ++et)
          dqt[et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr(sk, et, s4, lane), fs, dqt[et], 0, 0, 0);
      }
    }
    dma_barrier();  // the next tile has landed; every wave is done with this one
  }
  float amx = 0.f;  // max |stored dQ value| of the lane (fp8 scale partials; fused form only)
  if (myq < T) {
    if constexpr (FUSE) {
      amx = qknorm_rope_bwd_store(dqt, kScale, qh + (long long)myq * ld, rq[(rowbase + myq) * H + h], cs, T, myq, lh,
                                  dq_bf + (rowbase + myq) * ld_dq + h * 128);
    } else {
      float* dqr = dq_out + (rowbase + myq) * d + h * 128;
#pragma unroll
      for (int et = 0; et < 4; ++et)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int e = et * 32 + 8 * g + 4 * lh;
          *reinterpret_cast<float4*>(dqr + e) = make_float4(dqt[et][4 * g] * kScale, dqt[et][4 * g + 1] * kScale,
                                                            dqt[et][4 * g + 2] * kScale, dqt[et][4 * g + 3] * kScale);
        }
    }
  }
  store_wave_amax(amax, ((long long)blockIdx.x + (long long)gridDim.x * blockIdx.y) * (DQ_NT / 64) + wave, amx);
}

}  // namespace

long long attn_fwd_amax_slots(int B, int H, int T) { return (long long)((T + FQ - 1) / FQ) * B * H * 4; }

long long attn_bwd_amax_slots(int B, int H, int Hkv, int T) {
  return (long long)((T + DQ_Q - 1) / DQ_Q) * B * H * (DQ_NT / 64) +
         (long long)((T + K8_KEYS - 1) / K8_KEYS) * B * Hkv * (K8_NT / 64);
}

int launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, long long ld_qkv, uint16_t* out,
                    long long ld_out, float* lse, int B, int H, int Hkv, int T, int window, hipStream_t s,
                    bool lse_log2, float* amax) {
  if (B <= 0 || T <= 0) return 0;
  dim3 grid((T + FQ - 1) / FQ, B * H);
  const bool gen = Hkv != H || window >= 0;
  hipLaunchKernelGGL(gen ? attn_fwd_kernel<true> : attn_fwd_kernel<false>, grid, dim3(256), 0, s, q, k, v, ld_qkv, out,
                     ld_out, lse, H, Hkv, T, window, lse_log2 ? 1 : 0, amax);
  GS_LAUNCH_CHECK("attn_fwd");
  return 0;
}

int launch_attn_bwd_part(int part, const uint16_t* q, const uint16_t* k, const uint16_t* v, long long ld_qkv,
                         const uint16_t* out, const uint16_t* dout, long long ld_out, const float* lse, float* delta,
                         float* dq, uint16_t* dk, uint16_t* dv, long long ld_dkv, int B, int H, int Hkv, int T,
                         int window, hipStream_t s, const QkNormBwd* fuse) {
  if (B <= 0 || T <= 0) return 0;
  const bool gen = Hkv != H || window >= 0;
  const float* rq = fuse ? fuse->rq : nullptr;
  const float* rk = fuse ? fuse->rk : nullptr;
  const float* cs = fuse ? fuse->cs : nullptr;
  uint16_t* dq_bf = fuse ? fuse->dq : nullptr;
  float* amax = fuse ? fuse->amax : nullptr;  // dQ kernel's waves, then the dK/dV kernel's
  if (part == 0) {  // dQ, and delta for the dK/dV kernel
    auto kern = fuse ? (gen ? attn_bwd_q_kernel<true, true> : attn_bwd_q_kernel<false, true>)
                     : (gen ? attn_bwd_q_kernel<true, false> : attn_bwd_q_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3((T + DQ_Q - 1) / DQ_Q, B * H), dim3(DQ_NT), 0, s, q, k, v, ld_qkv, out, dout, ld_out,
                       lse, delta, dq, H, Hkv, T, window, dq_bf, ld_dkv, rq, cs, amax);
    GS_LAUNCH_CHECK("attn_bwd_q");
  } else {
    auto kern = fuse ? (gen ? attn_bwd_kv8_kernel<true, true> : attn_bwd_kv8_kernel<false, true>)
                     : (gen ? attn_bwd_kv8_kernel<true, false> : attn_bwd_kv8_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3((T + K8_KEYS - 1) / K8_KEYS, B * Hkv), dim3(K8_NT), 0, s, q, k, v, ld_qkv, dout,
                       ld_out, lse, delta, dk, dv, ld_dkv, H, Hkv, T, window, rk, cs,
                       amax ? amax + (long long)((T + DQ_Q - 1) / DQ_Q) * B * H * (DQ_NT / 64) : nullptr);
    GS_LAUNCH_CHECK("attn_bwd_kv");
  }
  return 0;
}

int launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, long long ld_qkv,
                    const uint16_t* out, const uint16_t* dout, long long ld_out, const float* lse, float* delta,
                    float* dq, uint16_t* dk, uint16_t* dv, long long ld_dkv, int B, int H, int Hkv, int T,
                    int window, hipStream_t s) {
  for (int part = 0; part < 2; ++part) {
    const int rc = launch_attn_bwd_part(part, q, k, v, ld_qkv, out, dout, ld_out, lse, delta, dq, dk, dv, ld_dkv, B,
                                        H, Hkv, T, window, s, nullptr);
    if (rc) return rc;
  }
  return 0;
}

}  // namespace gs
