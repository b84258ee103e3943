// Bandwidth-bound kernels of the step: embedding gather/scatter, RMSNorm,
// rotary embedding with QK normalisation, cross-entropy row reduction, loss
// mean, and the elementwise parts of the Muon update.
//
// Model passage (dev.to "¿Cómo Entrenar Tu Propio ChatGPT por $50?",
// "1. Modelo GPT"): rotary embeddings, QK normalisation, untied token
// embedding.  Muon passage ("2. Optimizador Muon"): momentum, normalised start
// of the Newton-Schulz iteration, apply.  Readings used here: gainless RMS
// norm with eps = 1e-6 inside the root; rotation of pairs (i, i + 64) by
// angle t * 10000^(-i/64); QK norm over each 128-wide head after rotation.
//
// Every kernel here streams its rows once: one wave64 per row (vectorised
// 16-byte accesses) so the row statistics reduce with wave shuffles only.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gs {

namespace {

constexpr float kEps = 1e-6f;
constexpr int kMaxD = 4096;              // 64 * 64 (largest supported depth)
constexpr int kMaxChunks = kMaxD / 4 / 64;  // float4 chunks per lane at d = 4096

inline int nblocks(long long n, int per) { return (int)((n + per - 1) / per); }

// ----------------------------------------------------------------------------
__global__ void fill_f32_kernel(float* p, long long n, float v) {
  long long i = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const long long stride = (long long)gridDim.x * blockDim.x * 4;
  for (; i < n; i += stride) {
    if (i + 3 < n && (((uintptr_t)(p + i)) & 15) == 0) {
      *reinterpret_cast<float4*>(p + i) = make_float4(v, v, v, v);
    } else {
      for (int j = 0; j < 4 && i + j < n; ++j) p[i + j] = v;
    }
  }
}

__global__ void cast_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst, long long n) {
  long long i = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const long long stride = (long long)gridDim.x * blockDim.x * 4;
  for (; i < n; i += stride) {
    if (i + 3 < n) {
      const float4 v = *reinterpret_cast<const float4*>(src + i);
      *reinterpret_cast<uint2*>(dst + i) = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
    } else {
      for (int j = 0; i + j < n; ++j) dst[i + j] = f2bf(src[i + j]);
    }
  }
}

// cos/sin of t * 10000^(-2i/128), computed in double precision
__global__ void rope_table_kernel(float* cs, int T) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * 64) return;
  const int t = idx / 64, i = idx % 64;
  const double inv_freq = pow(10000.0, -(2.0 * i) / 128.0);
  const double ang = (double)t * inv_freq;
  cs[idx] = (float)cos(ang);
  cs[T * 64 + idx] = (float)sin(ang);
}

// x[n, :] = wte[ids[b, t], :] for n = b*T + t (bf16 -> fp32, exact); an id
// outside [0, V) reads nothing and gives a zero row
__global__ void __launch_bounds__(256) embed_fwd_kernel(const int* __restrict__ ids, const uint16_t* __restrict__ wte,
                                 float* __restrict__ x, int B, int T, int d, int V) {
  const int lane = threadIdx.x & 63;
  const long long n = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= (long long)B * T) return;
  const int b = (int)(n / T), t = (int)(n % T);
  const long long id = ids[(long long)b * (T + 1) + t];
  const bool ok = id >= 0 && id < V;
  const uint16_t* src = wte + (ok ? id : 0) * d;
  float* dst = x + n * d;
  for (int c = lane; c < d / 8; c += 64) {
    const uint4 w = ok ? *reinterpret_cast<const uint4*>(src + c * 8) : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<float4*>(dst + c * 8) = make_float4(lo_bf(w.x), hi_bf(w.x), lo_bf(w.y), hi_bf(w.y));
    *reinterpret_cast<float4*>(dst + c * 8 + 4) = make_float4(lo_bf(w.z), hi_bf(w.z), lo_bf(w.w), hi_bf(w.w));
  }
}

// Embedding backward without atomics, deterministic: a stable counting sort
// of the token ids (tokens of one id keep their order), then one wave per
// vocabulary row sums its tokens' gradient rows in token order.
//   emb_rank:   per 1024-token block, each token's rank among the block's
//               tokens of its id, and the block's count of each id (written
//               by the id's last token in the block; the array is zeroed first)
//   emb_blocks: per id, exclusive prefix of its counts over the blocks (in
//               place) and its total
//   emb_scan:   exclusive prefix of the totals over the ids (one workgroup)
//   emb_place:  token n goes to position off[id] + block prefix + rank
//   emb_gather: dwte[v] (+)= sum of g over the tokens of v
// Ids outside [0, V) take no part: they are neither counted nor placed.
constexpr int kEmbBlk = 1024;
__device__ __forceinline__ int token_id(const int* ids, long long n, int T) {
  return ids[(n / T) * (T + 1) + n % T];
}

__global__ void __launch_bounds__(kEmbBlk) emb_rank_kernel(const int* __restrict__ ids, long long N, int T, int V,
                                                           int* __restrict__ blockcnt, int* __restrict__ rank) {
  __shared__ int sid[kEmbBlk];
  const long long n0 = (long long)blockIdx.x * kEmbBlk;
  const int cnt = (int)min((long long)kEmbBlk, N - n0);
  const int t = threadIdx.x;
  int tid_ = t < cnt ? token_id(ids, n0 + t, T) : -1;
  sid[t] = (tid_ >= 0 && tid_ < V) ? tid_ : -1;
  __syncthreads();
  if (t >= cnt) return;
  const int id = sid[t];
  if (id < 0) return;
  int r = 0;
  bool last = true;
  for (int j = 0; j < cnt; ++j) {
    const bool same = sid[j] == id;
    r += (same && j < t) ? 1 : 0;
    last = last && !(same && j > t);
  }
  rank[n0 + t] = r;
  if (last) blockcnt[(long long)blockIdx.x * V + id] = r + 1;
}

__global__ void __launch_bounds__(256) emb_blocks_kernel(int* __restrict__ blockcnt, int nb, int V,
                                                         int* __restrict__ total) {
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  int run = 0;
  for (int b = 0; b < nb; ++b) {
    const int c = blockcnt[(long long)b * V + v];
    blockcnt[(long long)b * V + v] = run;
    run += c;
  }
  total[v] = run;
}

// off[v] = sum of total[u] for u < v, off[V] = N; one workgroup of 1024
__global__ void __launch_bounds__(1024) emb_scan_kernel(const int* __restrict__ total, int V, int* __restrict__ off) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (V + 1023) / 1024;
  const int beg = min(V, t * per), end = min(V, beg + per);
  int s = 0;
  for (int v = beg; v < end; ++v) s += total[v];
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan over the 1024 partial sums
    const int x = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += x;
    __syncthreads();
  }
  int run = part[t] - s;
  for (int v = beg; v < end; ++v) {
    off[v] = run;
    run += total[v];
  }
  if (t == 1023) off[V] = part[1023];
}

__global__ void __launch_bounds__(256) emb_place_kernel(const int* __restrict__ ids, long long N, int T, int V,
                                                        const int* __restrict__ blockcnt, const int* __restrict__ rank,
                                                        const int* __restrict__ off, int* __restrict__ perm) {
  const long long n = (long long)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int id = token_id(ids, n, T);
  if (id < 0 || id >= V) return;
  const long long b = n / kEmbBlk;
  perm[off[id] + blockcnt[b * V + id] + rank[n]] = (int)n;
}

// one wave per vocabulary row; d a multiple of 4
__global__ void __launch_bounds__(256) emb_gather_kernel(const int* __restrict__ off, const int* __restrict__ perm,
                                                         const float* __restrict__ g, float* __restrict__ dwte, int V,
                                                         int d, int accumulate) {
  const int lane = threadIdx.x & 63;
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= V) return;
  const int beg = off[v], end = off[v + 1];
  float* dst = dwte + (long long)v * d;
  for (int c = lane; c < d / 4; c += 64) {
    float4 a = accumulate ? *reinterpret_cast<const float4*>(dst + c * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = beg; j < end; ++j) {
      const float4 x = *reinterpret_cast<const float4*>(g + (long long)perm[j] * d + c * 4);
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
    }
    *reinterpret_cast<float4*>(dst + c * 4) = a;
  }
}

// h = x * r, r = 1/sqrt(mean(x^2) + eps); one wave per row.  MC = float4
// chunks per lane (ceil(d / 256)): a compile-time count keeps the row in as
// few registers as it needs, so more waves fit per SIMD.
template <int MC>
__global__ void __launch_bounds__(256) rmsnorm_fwd_kernel(const float* __restrict__ x, uint16_t* __restrict__ h,
                                   float* __restrict__ r, long long N, int d, float* __restrict__ amax_part) {
  const int lane = threadIdx.x & 63;
  const long long n = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int nc = d / 4;
  const float* xr = x + n * d;
  float4 v[MC];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int c = i * 64 + lane;
    if (c < nc) {
      v[i] = *reinterpret_cast<const float4*>(xr + c * 4);
      ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    }
  }
  ss = wave_sum(ss);
  const float rr = 1.0f / sqrtf(ss / (float)d + kEps);
  uint16_t* hr = h + n * d;
  float amx = 0.f;
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int c = i * 64 + lane;
    if (c < nc) {
      const uint2 w = make_uint2(pack_bf2(v[i].x * rr, v[i].y * rr), pack_bf2(v[i].z * rr, v[i].w * rr));
      *reinterpret_cast<uint2*>(hr + c * 4) = w;
      if (amax_part)
        amx = fmaxf(amx, fmaxf(fmaxf(fabsf(lo_bf(w.x)), fabsf(hi_bf(w.x))), fmaxf(fabsf(lo_bf(w.y)), fabsf(hi_bf(w.y)))));
    }
  }
  if (amax_part) {  // launch-uniform: max |h| of this row (fp8 quantisation scale)
    amx = wave_max(amx);
    if (lane == 0) amax_part[n] = amx;
  }
  if (lane == 0) r[n] = rr;
}

// g += r * (dh - h * mean(dh * h)); g_bf = bf16(g); one wave per row (MC as
// in the forward).  dh is the bf16 output of a data-gradient product (DH16),
// or an fp32 sum of such products, rounded to bf16 as it is read.
template <int MC, bool DH16>
__global__ void __launch_bounds__(256) rmsnorm_bwd_kernel(const void* __restrict__ dhv, const uint16_t* __restrict__ h,
                                   const float* __restrict__ r, float* __restrict__ g,
                                   uint16_t* __restrict__ g_bf, long long N, int d, float* __restrict__ amax_part) {
  const int lane = threadIdx.x & 63;
  const long long n = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int nc = d / 4;
  float4 dv[MC], hv[MC];
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int c = i * 64 + lane;
    if (c < nc) {
      if constexpr (DH16) {
        const uint2 q = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(dhv) + n * d + c * 4);
        dv[i] = make_float4(lo_bf(q.x), hi_bf(q.x), lo_bf(q.y), hi_bf(q.y));
      } else {
        const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(dhv) + n * d + c * 4);
        dv[i] = make_float4(bf2f(f2bf(f.x)), bf2f(f2bf(f.y)), bf2f(f2bf(f.z)), bf2f(f2bf(f.w)));
      }
      const uint2 w = *reinterpret_cast<const uint2*>(h + n * d + c * 4);
      hv[i] = make_float4(lo_bf(w.x), hi_bf(w.x), lo_bf(w.y), hi_bf(w.y));
      dot += dv[i].x * hv[i].x + dv[i].y * hv[i].y + dv[i].z * hv[i].z + dv[i].w * hv[i].w;
    }
  }
  dot = wave_sum(dot) / (float)d;
  const float rr = r[n];
  float amx = 0.f;
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int c = i * 64 + lane;
    if (c < nc) {
      float4 gv = *reinterpret_cast<const float4*>(g + n * d + c * 4);
      gv.x += rr * (dv[i].x - hv[i].x * dot);
      gv.y += rr * (dv[i].y - hv[i].y * dot);
      gv.z += rr * (dv[i].z - hv[i].z * dot);
      gv.w += rr * (dv[i].w - hv[i].w * dot);
      st_nt(g + n * d + c * 4, gv);  // read again only by the next norm backward
      const uint2 w = make_uint2(pack_bf2(gv.x, gv.y), pack_bf2(gv.z, gv.w));
      *reinterpret_cast<uint2*>(g_bf + n * d + c * 4) = w;
      if (amax_part)
        amx = fmaxf(amx, fmaxf(fmaxf(fabsf(lo_bf(w.x)), fabsf(hi_bf(w.x))), fmaxf(fabsf(lo_bf(w.y)), fabsf(hi_bf(w.y)))));
    }
  }
  if (amax_part) {  // launch-uniform: max |g_bf| of this row (fp8 quantisation scale)
    amx = wave_max(amx);
    if (lane == 0) amax_part[n] = amx;
  }
}

// Cross-entropy gradient of one vocabulary chunk (columns c0 .. c0+nv-1) from
// the exponentials the forward kept, one wave per row: e = exp(z - mx_g) (fp16)
// with mx_g the row max of each group of cw columns (the .x of that group's
// (max, sum) partial), so softmax(z)[v] = e[v] exp(mx_g - lse).
// dz[n, j] = bf16(scale (softmax[c0 + j] - [c0 + j == target(n)])); the target
// of token n = b T + t is ids[b, t + 1].  Rows are ld elements apart in e and
// dz (ld % 4 == 0; cw and c0 multiples of 4).
__global__ void __launch_bounds__(256) ce_dz_kernel(const uint16_t* __restrict__ e, uint16_t* __restrict__ dz,
                                                    const float2* __restrict__ part, int nparts, int cw, int c0,
                                                    const float* __restrict__ lse, const int* __restrict__ ids, int T,
                                                    long long N, int nv, int ld, float scale) {
  const int lane = threadIdx.x & 63;
  const long long n = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int b = (int)(n / T), t = (int)(n % T);
  const int tgt = ids[(long long)b * (T + 1) + t + 1] - c0;  // chunk column of the target (may be outside)
  const float l = lse[n];
  const float2* pr = part + n * nparts;
  const uint16_t* er = e + n * ld;
  uint16_t* row = dz + n * ld;
  typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
  for (int c = lane * 4; c < nv; c += 256) {
    const float f = __expf(pr[(c0 + c) / cw].x - l);  // the 4 columns share a group
    if (c + 3 < nv) {
      const h4_t h = *reinterpret_cast<const h4_t*>(er + c);
      const float o0 = ((float)h[0] * f - (c == tgt ? 1.f : 0.f)) * scale;
      const float o1 = ((float)h[1] * f - (c + 1 == tgt ? 1.f : 0.f)) * scale;
      const float o2 = ((float)h[2] * f - (c + 2 == tgt ? 1.f : 0.f)) * scale;
      const float o3 = ((float)h[3] * f - (c + 3 == tgt ? 1.f : 0.f)) * scale;
      *reinterpret_cast<uint2*>(row + c) = make_uint2(pack_bf2(o0, o1), pack_bf2(o2, o3));
    } else {
      for (int j = c; j < nv; ++j) {
        const float ej = (float)*reinterpret_cast<const _Float16*>(er + j);
        row[j] = f2bf((ej * __expf(pr[(c0 + j) / cw].x - l) - (j == tgt ? 1.f : 0.f)) * scale);
      }
    }
  }
}

// lse = log-sum-exp over the per-tile (max, sum exp) partials; loss = lse - z[target]
__global__ void __launch_bounds__(256) ce_reduce_kernel(const float2* __restrict__ part, int nparts, const float* __restrict__ zt,
                                 float* __restrict__ lse, float* __restrict__ row_loss,
                                 float* __restrict__ lse_out, long long N) {
  const int lane = threadIdx.x & 63;
  const long long n = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const float2* p = part + n * nparts;
  float m = -INFINITY;
  for (int i = lane; i < nparts; i += 64) m = fmaxf(m, p[i].x);
  m = wave_max(m);
  float s = 0.f;
  for (int i = lane; i < nparts; i += 64) s += p[i].y * __expf(p[i].x - m);
  s = wave_sum(s);
  if (lane == 0) {
    const float l = m + logf(s);
    lse[n] = l;
    row_loss[n] = l - zt[n];
    if (lse_out) lse_out[n] = l;
  }
}

// loss = mean(row_loss), one block, double accumulation (deterministic)
__global__ void loss_mean_kernel(const float* __restrict__ row_loss, float* __restrict__ loss, long long N) {
  __shared__ double red[1024 / 64];
  double s = 0.0;
  for (long long i = threadIdx.x; i < N; i += blockDim.x) s += (double)row_loss[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < (int)(blockDim.x / 64); ++i) t += red[i];
    loss[0] = (float)(t / (double)N);
  }
}

// out = beta * out + sum of nsplit partials (stride elements apart); optional
// bf16 copy; out may be null (bf16 copy only, beta 0)
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int nsplit, long long stride,
                                     float* __restrict__ out, uint16_t* __restrict__ out_bf, long long n, float beta) {
  long long i = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const long long step = (long long)gridDim.x * blockDim.x * 4;
  for (; i < n; i += step) {
    if (i + 3 < n) {
      float4 acc = beta != 0.f ? *reinterpret_cast<const float4*>(out + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      if (beta != 0.f && beta != 1.f) { acc.x *= beta; acc.y *= beta; acc.z *= beta; acc.w *= beta; }
      for (int sp = 0; sp < nsplit; ++sp) {
        const float4 v = *reinterpret_cast<const float4*>(part + sp * stride + i);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      if (out) *reinterpret_cast<float4*>(out + i) = acc;
      if (out_bf) *reinterpret_cast<uint2*>(out_bf + i) = make_uint2(pack_bf2(acc.x, acc.y), pack_bf2(acc.z, acc.w));
    } else {
      for (long long j = i; j < n; ++j) {
        float a = beta != 0.f ? beta * out[j] : 0.f;
        for (int sp = 0; sp < nsplit; ++sp) a += part[sp * stride + j];
        if (out) out[j] = a;
        if (out_bf) out_bf[j] = f2bf(a);
      }
    }
  }
}

// ------------------------ symmetric matrix mirror ---------------------------
// C[b][i][j] = C[b][j][i] for i > j: 64 x 64 blocks (bi, bj), bi >= bj, of
// the lower triangle, each read from its mirror block (bj, bi) through LDS.
// Reads touch only elements with i < j (or the block's own upper part on the
// diagonal) and writes only i > j, so no element is both read and written.
// bf16 n x n matrices, n a multiple of 8 (so 8-element chunks lie wholly
// inside or outside).  Off-diagonal blocks move 16-byte chunks: the source
// block is read row-wise into LDS and each thread writes 8 consecutive
// elements of a destination row (a column of the source block); diagonal
// blocks copy element by element where i > j.
constexpr int kMirP = 72;  // LDS row pitch (elements) of the 64 x 64 block
__global__ void __launch_bounds__(256) sym_mirror_bf16_kernel(uint16_t* __restrict__ C, int n, long long ld,
                                                              long long stride) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kMirP];
  // block index -> (bi, bj), bi >= bj, row by row of the lower triangle
  const int x = blockIdx.x;
  int bi = (int)((sqrtf(8.f * x + 1.f) - 1.f) * 0.5f);
  while (bi * (bi + 1) / 2 > x) --bi;
  while ((bi + 1) * (bi + 2) / 2 <= x) ++bi;
  const int bj = x - bi * (bi + 1) / 2;
  uint16_t* c = C + (long long)blockIdx.y * stride;
  const int r0 = bj * 64, c0 = bi * 64;  // source block: rows r0.., columns c0..
  // source rows as 16-byte chunks: 64 rows x 8 chunks, two per thread
  for (int e = threadIdx.x; e < 512; e += 256) {
    const int rr = e >> 3, ch = (e & 7) * 8;
    const int gr = r0 + rr, gc = c0 + ch;
    if (gr < n && gc < n)
      *reinterpret_cast<uint4*>(tile + rr * kMirP + ch) = *reinterpret_cast<const uint4*>(c + (long long)gr * ld + gc);
  }
  __syncthreads();
  if (bi > bj) {
    // destination row c0 + rr, columns r0 + ch .. + 7 = tile column rr, rows ch .. ch + 7
    for (int e = threadIdx.x; e < 512; e += 256) {
      const int rr = e >> 3, ch = (e & 7) * 8;
      const int gi = c0 + rr, gj = r0 + ch;
      if (gi < n && gj < n) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[k] = (uint32_t)tile[(ch + 2 * k) * kMirP + rr] | ((uint32_t)tile[(ch + 2 * k + 1) * kMirP + rr] << 16);
        *reinterpret_cast<uint4*>(c + (long long)gi * ld + gj) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  } else {
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int rr = e >> 6, cc = e & 63;  // destination row c0 + rr, column r0 + cc
      const int gi = c0 + rr, gj = r0 + cc;
      if (gi < n && gj < n && gi > gj) c[(long long)gi * ld + gj] = tile[cc * kMirP + rr];
    }
  }
}

// ---------------------------- Muon elementwise ------------------------------
// Momentum and the Frobenius partials in one pass: M <- mu M + G over chunk
// blk of matrix b, partial[b * nblk + blk] = sum of squares of the new M
// (per a multiple of 4; float4 accesses, two in flight per thread)
__global__ void __launch_bounds__(256) momentum_frob_kernel(float* __restrict__ M, const float* __restrict__ G,
                                                            float mu, float* __restrict__ partial, long long per,
                                                            int nblk) {
  const int b = blockIdx.y, blk = blockIdx.x;
  const long long per4 = per / 4;
  const long long chunk = (per4 + nblk - 1) / nblk;
  const long long beg = blk * chunk, end = min(per4, beg + chunk);
  float4* m4 = reinterpret_cast<float4*>(M + (long long)b * per);
  const float4* g4 = reinterpret_cast<const float4*>(G + (long long)b * per);
  float s0 = 0.f, s1 = 0.f;
  long long i = beg + threadIdx.x;
  for (; i + 256 < end; i += 2 * 256) {
    float4 a = m4[i], c = m4[i + 256];
    const float4 ga = g4[i], gc = g4[i + 256];
    a.x = mu * a.x + ga.x; a.y = mu * a.y + ga.y; a.z = mu * a.z + ga.z; a.w = mu * a.w + ga.w;
    c.x = mu * c.x + gc.x; c.y = mu * c.y + gc.y; c.z = mu * c.z + gc.z; c.w = mu * c.w + gc.w;
    m4[i] = a;
    m4[i + 256] = c;
    s0 += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    s1 += c.x * c.x + c.y * c.y + c.z * c.z + c.w * c.w;
  }
  for (; i < end; i += 256) {
    float4 a = m4[i];
    const float4 ga = g4[i];
    a.x = mu * a.x + ga.x; a.y = mu * a.y + ga.y; a.z = mu * a.z + ga.z; a.w = mu * a.w + ga.w;
    m4[i] = a;
    s0 += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
  }
  float s = s0 + s1;
  __shared__ float red[4];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) partial[(long long)b * nblk + blk] = red[0] + red[1] + red[2] + red[3];
}

// partial[b * nblk + blk] = sum of squares of chunk blk of matrix b; per is a
// multiple of 4 (the matrices' sides are multiples of 8), read as float4 with
// four loads in flight per thread
__global__ void __launch_bounds__(256) frob_partial_kernel(const float* __restrict__ X, float* __restrict__ partial,
                                                           long long per, int nblk) {
  const int b = blockIdx.y, blk = blockIdx.x;
  const long long per4 = per / 4;
  const long long chunk = (per4 + nblk - 1) / nblk;
  const long long beg = blk * chunk, end = min(per4, beg + chunk);
  const float4* x = reinterpret_cast<const float4*>(X + (long long)b * per);
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  long long i = beg + threadIdx.x;
  for (; i + 3 * 256 < end; i += 4 * 256) {
    const float4 a = x[i], c = x[i + 256], d = x[i + 512], e = x[i + 768];
    s0 += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    s1 += c.x * c.x + c.y * c.y + c.z * c.z + c.w * c.w;
    s2 += d.x * d.x + d.y * d.y + d.z * d.z + d.w * d.w;
    s3 += e.x * e.x + e.y * e.y + e.z * e.z + e.w * e.w;
  }
  for (; i < end; i += 256) {
    const float4 a = x[i];
    s0 += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
  }
  float s = (s0 + s1) + (s2 + s3);
  __shared__ float red[4];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) partial[(long long)b * nblk + blk] = red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ float frob_norm(const float* partial, int b, int nblk) {
  double s = 0.0;
  for (int i = 0; i < nblk; ++i) s += (double)partial[(long long)b * nblk + i];
  return (float)sqrt(s);
}

// 64x64 output tiles, 256 threads; TR: out[i][j] = in[j][i]; X (the fp32
// copy) nullable: the iteration reads only the bf16 one
template <bool TR>
__global__ void ns_init_kernel(const float* __restrict__ src, const float* __restrict__ partial, int nblk,
                               float* __restrict__ X, uint16_t* __restrict__ Xb, int rows, int cols,
                               float eps) {
  // output oriented [l, s]: l = max(rows, cols), s = min
  const int b = blockIdx.z;
  const int lr = TR ? cols : rows, ls = TR ? rows : cols;
  const float inv = 1.0f / (frob_norm(partial, b, nblk) + eps);
  const float* in = src + (long long)b * rows * cols;
  float* out = X + (long long)b * rows * cols;
  uint16_t* outb = Xb + (long long)b * rows * cols;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  __shared__ float tile[64][65];
  if (TR) {
    // in is [rows, cols] = [ls, lr]; out[i][j] = in[j][i]; 4 consecutive
    // elements per thread on both sides (lr, ls multiples of 8)
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
      const int jj = e / 16, ii = (e % 16) * 4;  // read in[j0+jj][i0+ii ..] coalesced along ii
      const int gj = j0 + jj, gi = i0 + ii;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (gj < ls && gi < lr) v = *reinterpret_cast<const float4*>(in + (long long)gj * lr + gi);
      tile[jj][ii] = v.x; tile[jj][ii + 1] = v.y; tile[jj][ii + 2] = v.z; tile[jj][ii + 3] = v.w;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
      const int ii = e / 16, jj = (e % 16) * 4;
      const int gi = i0 + ii, gj = j0 + jj;
      if (gi < lr && gj < ls) {
        const long long o = (long long)gi * ls + gj;
        const float4 v = make_float4(tile[jj][ii] * inv, tile[jj + 1][ii] * inv, tile[jj + 2][ii] * inv,
                                     tile[jj + 3][ii] * inv);
        if (X) *reinterpret_cast<float4*>(out + o) = v;
        *reinterpret_cast<uint2*>(outb + o) = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
      }
    }
  } else {
    // 4 consecutive elements per thread (ls % 8 == 0: rows of 16-byte chunks)
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
      const int ii = e / 16, jj = (e % 16) * 4;
      const int gi = i0 + ii, gj = j0 + jj;
      if (gi < lr && gj < ls) {
        const long long o = (long long)gi * ls + gj;
        float4 v = *reinterpret_cast<const float4*>(in + o);
        v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
        if (X) *reinterpret_cast<float4*>(out + o) = v;
        *reinterpret_cast<uint2*>(outb + o) = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// NorMuon: per-neuron sums of squares of the orthogonalised update X (stored
// [l, s] per matrix), then per matrix the second-moment EMA, the step sizes
// and the norm ratio folded into one scale per neuron
// ---------------------------------------------------------------------------
constexpr int kNmRows = 256;  // stored rows per workgroup of the column statistic

// part[w] = sum of squares of stored row w (all matrices' rows in sequence);
// one wave per row, 16-byte loads (s % 4 == 0)
__global__ void __launch_bounds__(256) nm_rowsq_kernel(const uint16_t* __restrict__ X, float* __restrict__ part,
                                                       int sm, long long nrows) {
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= nrows) return;
  const uint16_t* x = X + w * sm;
  float acc = 0.f;
  for (int c = lane * 4; c < sm; c += 256) {
    const uint2 q = *reinterpret_cast<const uint2*>(x + c);
    const float a = lo_bf(q.x), b = hi_bf(q.x), e = lo_bf(q.y), f = hi_bf(q.y);
    acc += a * a + b * b + e * e + f * f;
  }
  acc = wave_sum(acc);
  if (lane == 0) part[w] = acc;
}

// part[(b nch + ch) s + c] = sum over stored rows ch*kNmRows .. of X[b][r][c]^2;
// a workgroup covers 64 columns (one per lane) and 4 interleaved row groups
__global__ void __launch_bounds__(256) nm_colsq_kernel(const uint16_t* __restrict__ X, float* __restrict__ part, int l,
                                                       int sm, int nch) {
  const int b = blockIdx.z, ch = blockIdx.y;
  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const int r0 = ch * kNmRows, r1 = min(l, r0 + kNmRows);
  float acc = 0.f;
  if (c < sm) {
    const uint16_t* x = X + (long long)b * l * sm + c;
    for (int r = r0 + g; r < r1; r += 4) {
      const float v = bf2f(x[(long long)r * sm]);
      acc += v * v;
    }
  }
  __shared__ float red[4][64];
  red[g][lane] = acc;
  __syncthreads();
  if (g == 0 && c < sm) part[((long long)b * nch + ch) * sm + c] = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
}

// one workgroup per matrix: vm_i = (sum over chunks) / n; V_i <- beta2 V_i +
// (1 - beta2) vm_i; step_i = 1 / (sqrt(V_i) + eps);
// scale_i = step_i sqrt(sum vm) / max(sqrt(sum vm step^2), 1e-10)
__global__ void __launch_bounds__(256) nm_finalize_kernel(const float* __restrict__ part, int nch, int nneur,
                                                          float inv_n, float* __restrict__ V,
                                                          float* __restrict__ scale, float beta2, float eps) {
  const int b = blockIdx.x;
  const float* p = part + (long long)b * nch * nneur;
  float* v = V + (long long)b * nneur;
  float* sc = scale + (long long)b * nneur;
  double s0 = 0.0, s1 = 0.0;
  for (int i = threadIdx.x; i < nneur; i += 256) {
    float ss = 0.f;
    for (int ch = 0; ch < nch; ++ch) ss += p[(long long)ch * nneur + i];
    const float vm = ss * inv_n;
    const float vn = beta2 * v[i] + (1.f - beta2) * vm;
    v[i] = vn;
    const float st = 1.f / (sqrtf(vn) + eps);
    sc[i] = st;
    s0 += vm;
    s1 += (double)vm * st * st;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    s0 += __shfl_xor(s0, o, 64);
    s1 += __shfl_xor(s1, o, 64);
  }
  __shared__ double red[2][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { red[0][wave] = s0; red[1][wave] = s1; }
  __syncthreads();
  const double t0 = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  const double t1 = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const float ratio = (float)(sqrt(t0) / fmax(sqrt(t1), 1e-10));
  for (int i = threadIdx.x; i < nneur; i += 256) sc[i] *= ratio;  // entries this thread wrote
}

// output tiles over W [rows, cols]; X oriented [l, s] (transposed when TR);
// nsc (nullable): NorMuon scale per row (nm_rows) or per column of W
template <bool TR, bool VEC>
__global__ void muon_apply_kernel(const uint16_t* __restrict__ X, float* __restrict__ W, uint16_t* __restrict__ Wb,
                                  float* __restrict__ O_out, int rows, int cols, float lr, float wd,
                                  const float* __restrict__ nsc, int nm_rows) {
  const int b = blockIdx.z;
  const uint16_t* x = X + (long long)b * rows * cols;
  const long long base = (long long)b * rows * cols;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  __shared__ float tile[64][65];
  if (TR) {
    // X is [cols, rows]; O[r][c] = X[c][r]
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int cc = e / 64, rr = e % 64;
      const int gc = c0 + cc, gr = r0 + rr;
      tile[cc][rr] = (gc < cols && gr < rows) ? bf2f(x[(long long)gc * rows + gr]) : 0.f;
    }
    __syncthreads();
  }
  const float decay = 1.f - lr * wd;
  if (VEC) {
    // 4 consecutive columns per thread: cols % 8 == 0 and 16-byte aligned
    // W, O_out (8-byte aligned X, Wb), checked by the launcher
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
      const int rr = e / 16, c4 = (e % 16) * 4;
      const int gr = r0 + rr, gc = c0 + c4;
      if (gr < rows && gc < cols) {
        const long long idx = (long long)gr * cols + gc;
        float o[4];
        if (TR) {
          o[0] = tile[c4][rr]; o[1] = tile[c4 + 1][rr]; o[2] = tile[c4 + 2][rr]; o[3] = tile[c4 + 3][rr];
        } else {
          const uint2 q = *reinterpret_cast<const uint2*>(x + idx);
          o[0] = lo_bf(q.x); o[1] = hi_bf(q.x); o[2] = lo_bf(q.y); o[3] = hi_bf(q.y);
        }
        if (nsc) {
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] *= nm_rows ? nsc[(long long)b * rows + gr] : nsc[(long long)b * cols + gc + j];
        }
        if (O_out) *reinterpret_cast<float4*>(O_out + base + idx) = make_float4(o[0], o[1], o[2], o[3]);
        if (W) {
          float4 w = *reinterpret_cast<const float4*>(W + base + idx);
          w.x = w.x * decay - lr * o[0]; w.y = w.y * decay - lr * o[1];
          w.z = w.z * decay - lr * o[2]; w.w = w.w * decay - lr * o[3];
          st_nt(W + base + idx, w);  // the weights are read by the next step
          if (Wb) st_nt(Wb + base + idx, make_uint2(pack_bf2(w.x, w.y), pack_bf2(w.z, w.w)));
        }
      }
    }
    return;
  }
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int rr = e / 64, cc = e % 64;
    const int gr = r0 + rr, gc = c0 + cc;
    if (gr < rows && gc < cols) {
      const long long idx = (long long)gr * cols + gc;
      float o = TR ? tile[cc][rr] : bf2f(x[idx]);
      if (nsc) o *= nm_rows ? nsc[(long long)b * rows + gr] : nsc[(long long)b * cols + gc];
      if (O_out) O_out[base + idx] = o;
      if (W) {
        const float w = W[base + idx] * decay - lr * o;
        W[base + idx] = w;
        if (Wb) Wb[base + idx] = f2bf(w);
      }
    }
  }
}

// AdamW with decoupled weight decay on 4 parameters per thread (n % 4 == 0,
// 16-byte aligned arrays): g = gs G; m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
// W = W (1 - lr wd) - lr (m / bc1) / (sqrt(v / bc2) + eps); Wb = bf16(W)
__global__ void __launch_bounds__(256) adamw_kernel(float* __restrict__ W, uint16_t* __restrict__ Wb,
                                                    const float* __restrict__ G, float* __restrict__ M,
                                                    float* __restrict__ V, long long n4, float lr, float b1,
                                                    float b2, float eps, float wd, float inv_bc1, float inv_bc2,
                                                    float gs) {
  const float decay = 1.f - lr * wd;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
    const float4 g4 = reinterpret_cast<const float4*>(G)[i];
    float4 m4 = reinterpret_cast<float4*>(M)[i];
    float4 v4 = reinterpret_cast<float4*>(V)[i];
    float4 w4 = reinterpret_cast<float4*>(W)[i];
    float g[4] = {g4.x, g4.y, g4.z, g4.w}, m[4] = {m4.x, m4.y, m4.z, m4.w};
    float v[4] = {v4.x, v4.y, v4.z, v4.w}, w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float gj = g[j] * gs;
      m[j] = b1 * m[j] + (1.f - b1) * gj;
      v[j] = b2 * v[j] + (1.f - b2) * gj * gj;
      w[j] = w[j] * decay - lr * (m[j] * inv_bc1) / (sqrtf(v[j] * inv_bc2) + eps);
    }
    // the state and weights are read by the next step
    st_nt(M + 4 * i, make_float4(m[0], m[1], m[2], m[3]));
    st_nt(V + 4 * i, make_float4(v[0], v[1], v[2], v[3]));
    st_nt(W + 4 * i, make_float4(w[0], w[1], w[2], w[3]));
    if (Wb) st_nt(Wb + 4 * i, make_uint2(pack_bf2(w[0], w[1]), pack_bf2(w[2], w[3])));
  }
}

}  // namespace

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
int launch_fill_f32(float* p, long long n, float v, hipStream_t s) {
  if (n <= 0) return 0;
  const int blocks = (int)std::min<long long>(nblocks(n, 1024), 8192);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks), dim3(256), 0, s, p, n, v);
  GS_LAUNCH_CHECK("fill_f32");
  return 0;
}

int launch_cast_bf16(const float* src, uint16_t* dst, long long n, hipStream_t s) {
  if (n <= 0) return 0;
  const int blocks = (int)std::min<long long>(nblocks(n, 1024), 16384);
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(blocks), dim3(256), 0, s, src, dst, n);
  GS_LAUNCH_CHECK("cast_bf16");
  return 0;
}

int launch_rope_table(float* cs, int T, hipStream_t s) {
  hipLaunchKernelGGL(rope_table_kernel, dim3(nblocks((long long)T * 64, 256)), dim3(256), 0, s, cs, T);
  GS_LAUNCH_CHECK("rope_table");
  return 0;
}

int launch_embed_fwd(const int* ids, const uint16_t* wte, float* x, int B, int T, int d, int V, hipStream_t s) {
  hipLaunchKernelGGL(embed_fwd_kernel, dim3(nblocks((long long)B * T, 4)), dim3(256), 0, s, ids, wte, x, B, T, d, V);
  GS_LAUNCH_CHECK("embed_fwd");
  return 0;
}

size_t embed_bwd_workspace(long long N, int V) {
  const long long nb = (N + kEmbBlk - 1) / kEmbBlk;
  return (size_t)(nb * V + V + (V + 1) + 2 * N) * 4;
}

int launch_embed_sort(const int* ids, int B, int T, int V, void* ws, hipStream_t s) {
  const long long N = (long long)B * T;
  if (N <= 0 || V <= 0) return 0;
  const int nb = (int)((N + kEmbBlk - 1) / kEmbBlk);
  int* blockcnt = static_cast<int*>(ws);
  int* total = blockcnt + (long long)nb * V;
  int* off = total + V;
  int* rank = off + V + 1;
  int* perm = rank + N;
  {
    const int rc = launch_fill_f32(reinterpret_cast<float*>(blockcnt), (long long)nb * V, 0.f, s);  // int 0 = float 0
    if (rc) return rc;
  }
  hipLaunchKernelGGL(emb_rank_kernel, dim3(nb), dim3(kEmbBlk), 0, s, ids, N, T, V, blockcnt, rank);
  GS_LAUNCH_CHECK("emb_rank");
  hipLaunchKernelGGL(emb_blocks_kernel, dim3((V + 255) / 256), dim3(256), 0, s, blockcnt, nb, V, total);
  GS_LAUNCH_CHECK("emb_blocks");
  hipLaunchKernelGGL(emb_scan_kernel, dim3(1), dim3(1024), 0, s, total, V, off);
  GS_LAUNCH_CHECK("emb_scan");
  hipLaunchKernelGGL(emb_place_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, ids, N, T, V, blockcnt,
                     rank, off, perm);
  GS_LAUNCH_CHECK("emb_place");
  return 0;
}

int launch_embed_gather(const float* g, float* dst, long long N, int d, int V, bool accumulate, const void* ws,
                        hipStream_t s) {
  if (N <= 0 || V <= 0) return 0;
  const int nb = (int)((N + kEmbBlk - 1) / kEmbBlk);
  const int* off = static_cast<const int*>(ws) + (long long)nb * V + V;
  const int* perm = off + V + 1 + N;
  hipLaunchKernelGGL(emb_gather_kernel, dim3((V + 3) / 4), dim3(256), 0, s, off, perm, g, dst, V, d,
                     accumulate ? 1 : 0);
  GS_LAUNCH_CHECK("emb_gather");
  return 0;
}

// one instantiation per chunk count 1 .. kMaxChunks (d <= 4096)
#define GS_MC_SWITCH(mc, CALL) \
  switch (mc) {                \
    case 1: CALL(1); break;    \
    case 2: CALL(2); break;    \
    case 3: CALL(3); break;    \
    case 4: CALL(4); break;    \
    case 5: CALL(5); break;    \
    case 6: CALL(6); break;    \
    case 7: CALL(7); break;    \
    case 8: CALL(8); break;    \
    case 9: CALL(9); break;    \
    case 10: CALL(10); break;  \
    case 11: CALL(11); break;  \
    case 12: CALL(12); break;  \
    case 13: CALL(13); break;  \
    case 14: CALL(14); break;  \
    case 15: CALL(15); break;  \
    default: CALL(16); break;  \
  }
static_assert(kMaxChunks == 16, "chunk-count switch");

int launch_rmsnorm_fwd(const float* x, uint16_t* h, float* r, long long N, int d, hipStream_t s, float* amax_part) {
  const int mc = (d / 4 + 63) / 64;
#define GS_RF(M) hipLaunchKernelGGL((rmsnorm_fwd_kernel<M>), dim3(nblocks(N, 4)), dim3(256), 0, s, x, h, r, N, d, amax_part)
  GS_MC_SWITCH(mc, GS_RF)
#undef GS_RF
  GS_LAUNCH_CHECK("rmsnorm_fwd");
  return 0;
}

int launch_rmsnorm_bwd(const void* dh, bool dh_bf16, const uint16_t* h, const float* r, float* g, uint16_t* g_bf,
                       long long N, int d, hipStream_t s, float* amax_part) {
  const int mc = (d / 4 + 63) / 64;
#define GS_RB(M)                                                                                              \
  if (dh_bf16)                                                                                                \
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<M, true>), dim3(nblocks(N, 4)), dim3(256), 0, s, dh, h, r, g, g_bf, N, d, \
                       amax_part);                                                                           \
  else                                                                                                        \
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<M, false>), dim3(nblocks(N, 4)), dim3(256), 0, s, dh, h, r, g, g_bf, N, d, \
                       amax_part);
  GS_MC_SWITCH(mc, GS_RB)
#undef GS_RB
  GS_LAUNCH_CHECK("rmsnorm_bwd");
  return 0;
}

int launch_ce_dz(const uint16_t* e, uint16_t* dz, const float* part, int nparts, int cw, int c0, const float* lse,
                 const int* ids, int T, long long N, int nv, int ld, float scale, hipStream_t s) {
  if (N <= 0 || nv <= 0) return 0;
  hipLaunchKernelGGL(ce_dz_kernel, dim3(nblocks(N, 4)), dim3(256), 0, s, e, dz, reinterpret_cast<const float2*>(part),
                     nparts, cw, c0, lse, ids, T, N, nv, ld, scale);
  GS_LAUNCH_CHECK("ce_dz");
  return 0;
}

int launch_ce_reduce(const float* part, int nparts, const float* zt, float* lse, float* row_loss,
                     float* lse_out, long long N, hipStream_t s) {
  hipLaunchKernelGGL(ce_reduce_kernel, dim3(nblocks(N, 4)), dim3(256), 0, s,
                     reinterpret_cast<const float2*>(part), nparts, zt, lse, row_loss, lse_out, N);
  GS_LAUNCH_CHECK("ce_reduce");
  return 0;
}

int launch_loss_mean(const float* row_loss, float* loss, long long N, hipStream_t s) {
  hipLaunchKernelGGL(loss_mean_kernel, dim3(1), dim3(1024), 0, s, row_loss, loss, N);
  GS_LAUNCH_CHECK("loss_mean");
  return 0;
}

int launch_splitk_reduce(const float* part, int nsplit, long long stride, float* out, uint16_t* out_bf, long long n,
                         float beta, hipStream_t s) {
  if (n <= 0) return 0;
  if (!out && (beta != 0.f || !out_bf)) {
    set_error("splitk_reduce: without an fp32 output beta must be 0 and the bf16 output given");
    return -1;
  }
  const int blocks = (int)std::min<long long>(nblocks(n, 1024), 8192);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, part, nsplit, stride, out, out_bf, n, beta);
  GS_LAUNCH_CHECK("splitk_reduce");
  return 0;
}

int launch_sym_mirror(uint16_t* C, int n, long long ld, long long stride, int count, hipStream_t s) {
  if (n <= 1 || count <= 0) return 0;
  const int nb = (n + 63) / 64;
  dim3 grid(nb * (nb + 1) / 2, count);
  if ((n % 8) || (ld % 8) || (stride % 8) || (reinterpret_cast<uintptr_t>(C) % 16)) {
    set_error("sym_mirror: bf16 matrices need n, ld, stride multiples of 8 and a 16-byte aligned base");
    return -3;
  }
  hipLaunchKernelGGL(sym_mirror_bf16_kernel, grid, dim3(256), 0, s, C, n, ld, stride);
  GS_LAUNCH_CHECK("sym_mirror");
  return 0;
}

int launch_momentum_frob(float* M, const float* G, float mu, float* partial, int count, long long per, int nblk,
                         hipStream_t s) {
  hipLaunchKernelGGL(momentum_frob_kernel, dim3(nblk, count), dim3(256), 0, s, M, G, mu, partial, per, nblk);
  GS_LAUNCH_CHECK("momentum_frob");
  return 0;
}

int launch_frob_partial(const float* X, float* partial, int count, long long per, int nblk, hipStream_t s) {
  hipLaunchKernelGGL(frob_partial_kernel, dim3(nblk, count), dim3(256), 0, s, X, partial, per, nblk);
  GS_LAUNCH_CHECK("frob_partial");
  return 0;
}

int launch_ns_init(const float* src, const float* partial, int nblk, float* X, uint16_t* Xb, int count,
                   int rows, int cols, float eps, hipStream_t s) {
  const bool tr = rows < cols;
  const int lr = tr ? cols : rows, ls = tr ? rows : cols;
  dim3 grid((ls + 63) / 64, (lr + 63) / 64, count);
  if (tr)
    hipLaunchKernelGGL(ns_init_kernel<true>, grid, dim3(256), 0, s, src, partial, nblk, X, Xb, rows, cols, eps);
  else
    hipLaunchKernelGGL(ns_init_kernel<false>, grid, dim3(256), 0, s, src, partial, nblk, X, Xb, rows, cols, eps);
  GS_LAUNCH_CHECK("ns_init");
  return 0;
}

int launch_adamw(float* W, uint16_t* Wb, const float* G, float* M, float* V, long long n, float lr, float b1,
                 float b2, float eps, float wd, float inv_bc1, float inv_bc2, float gs, hipStream_t s) {
  if (n <= 0) return 0;
  const long long n4 = n / 4;
  const int blocks = (int)std::min<long long>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(adamw_kernel, dim3(blocks), dim3(256), 0, s, W, Wb, G, M, V, n4, lr, b1, b2, eps, wd, inv_bc1,
                     inv_bc2, gs);
  GS_LAUNCH_CHECK("adamw");
  return 0;
}

int launch_normuon_scale(const uint16_t* X, float* part, float* V, float* scale, int count, int rows, int cols,
                         int per_row, float beta2, float eps, hipStream_t s) {
  const bool tr = rows < cols;
  const int l = tr ? cols : rows, sm = tr ? rows : cols;
  const int nneur = per_row ? rows : cols;
  const float inv_n = 1.f / (float)(per_row ? cols : rows);
  int nch = 1;
  if ((per_row != 0) != tr) {  // neurons are the stored rows
    const long long nr = (long long)count * l;
    hipLaunchKernelGGL(nm_rowsq_kernel, dim3((unsigned)((nr + 3) / 4)), dim3(256), 0, s, X, part, sm, nr);
    GS_LAUNCH_CHECK("nm_rowsq");
  } else {                     // neurons are the stored columns
    nch = (l + kNmRows - 1) / kNmRows;
    hipLaunchKernelGGL(nm_colsq_kernel, dim3((sm + 63) / 64, nch, count), dim3(256), 0, s, X, part, l, sm, nch);
    GS_LAUNCH_CHECK("nm_colsq");
  }
  hipLaunchKernelGGL(nm_finalize_kernel, dim3(count), dim3(256), 0, s, part, nch, nneur, inv_n, V, scale, beta2, eps);
  GS_LAUNCH_CHECK("nm_finalize");
  return 0;
}

long long normuon_part_floats(int count, int rows, int cols) {
  const int l = std::max(rows, cols), sm = std::min(rows, cols);
  return (long long)count * std::max<long long>(l, (long long)sm * ((l + kNmRows - 1) / kNmRows));
}

int launch_muon_apply(const uint16_t* X, float* W, uint16_t* Wb, float* O_out, int count, int rows, int cols,
                      float lr, float wd, const float* nsc, int nm_rows, hipStream_t s) {
  const bool tr = rows < cols;
  dim3 grid((cols + 63) / 64, (rows + 63) / 64, count);
  auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  const bool vec = cols % 4 == 0 && al(X, 8) && al(W, 16) && al(O_out, 16) && al(Wb, 8);
#define GS_MA(T_, V_) hipLaunchKernelGGL((muon_apply_kernel<T_, V_>), grid, dim3(256), 0, s, X, W, Wb, O_out, rows, \
                                         cols, lr, wd, nsc, nm_rows)
  if (tr) {
    if (vec) GS_MA(true, true); else GS_MA(true, false);
  } else {
    if (vec) GS_MA(false, true); else GS_MA(false, false);
  }
#undef GS_MA
  GS_LAUNCH_CHECK("muon_apply");
  return 0;
}

}  // namespace gs
