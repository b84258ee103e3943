// Record-model features of the step: smear, value embeddings, per-layer
// residual scaling and backout (dev.to "¿Cómo Entrenar Tu Propio ChatGPT por
// $50?", section "1. Modelo GPT (nanochat/gpt.py)": value embeddings in the
// ResFormer style and the three efficiency tricks; apidog.com/pt "Modelo
// GPT").  All of it is bandwidth-bound elementwise work: one wave per token
// row, 16-byte accesses, scalars read on the device from the bf16 parameter
// copy (no host round trip).  Scalar and gate gradients are per-workgroup
// partial sums reduced by reduce_partials_kernel (deterministic, no atomics);
// the value-embedding tables' gradients go through the token embedding's
// stable sort and gather, so they are deterministic too.  A token id outside
// [0, V) is never used as an index: its embedding rows count as zero.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gs {

namespace {

constexpr float kEps = 1e-6f;
constexpr int kMaxD = 4096;
constexpr int kMaxChunks = kMaxD / 4 / 64;
constexpr int kSmearCh = 24;   // embedding channels feeding the smear gate
constexpr int kVeCh = 32;      // attention-input channels feeding the value-embedding gate

inline int nblocks(long long n, int per) { return (int)((n + per - 1) / per); }

__device__ __forceinline__ float bfv(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }
__device__ __forceinline__ float sigm(float z) { return 1.f / (1.f + expf(-z)); }

// ---------------------------------------------------------------------------
// smear: x_t = e_t + gate_t e_{t-1}, gate_t = lam sigmoid(e_t[:24] . w) (t >= 1)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) smear_fwd_kernel(const int* __restrict__ ids, const uint16_t* __restrict__ wte,
                                                        const uint16_t* __restrict__ sw, const uint16_t* __restrict__ slam,
                                                        float* __restrict__ x, float* __restrict__ x0,
                                                        float* __restrict__ sig_out, int B, int T, int d, int V) {
  const int lane = threadIdx.x & 63;
  const long long n = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= (long long)B * T) return;
  const int b = (int)(n / T), t = (int)(n % T);
  const long long row = (long long)b * (T + 1) + t;
  const int id = ids[row], idp = t > 0 ? ids[row - 1] : id;
  const float ok = (id >= 0 && id < V) ? 1.f : 0.f, okp = (idp >= 0 && idp < V) ? 1.f : 0.f;
  const uint16_t* e = wte + (long long)(ok != 0.f ? id : 0) * d;
  // slam NULL: no smear (plain gather, optionally copied to x0)
  float z = (slam && lane < kSmearCh) ? ok * bfv(e + lane) * bfv(sw + lane) : 0.f;
  z = wave_sum(z);
  const float sg = sigm(z);
  const float gate = (slam && t > 0) ? bfv(slam) * sg * okp : 0.f;
  const uint16_t* ep = okp != 0.f ? wte + (long long)idp * d : e;
  float* xr = x + n * d;
  float* x0r = x0 ? x0 + n * d : nullptr;
  for (int c = lane; c < d / 8; c += 64) {
    const uint4 w = *reinterpret_cast<const uint4*>(e + c * 8);
    const uint4 p = *reinterpret_cast<const uint4*>(ep + c * 8);
    const float4 lo = make_float4(ok * lo_bf(w.x) + gate * lo_bf(p.x), ok * hi_bf(w.x) + gate * hi_bf(p.x),
                                  ok * lo_bf(w.y) + gate * lo_bf(p.y), ok * hi_bf(w.y) + gate * hi_bf(p.y));
    const float4 hi = make_float4(ok * lo_bf(w.z) + gate * lo_bf(p.z), ok * hi_bf(w.z) + gate * hi_bf(p.z),
                                  ok * lo_bf(w.w) + gate * lo_bf(p.w), ok * hi_bf(w.w) + gate * hi_bf(p.w));
    *reinterpret_cast<float4*>(xr + c * 8) = lo;
    *reinterpret_cast<float4*>(xr + c * 8 + 4) = hi;
    if (x0r) {
      *reinterpret_cast<float4*>(x0r + c * 8) = lo;
      *reinterpret_cast<float4*>(x0r + c * 8 + 4) = hi;
    }
  }
  if (lane == 0) sig_out[n] = sg;
}

// Backward of smear for token t (one wave): with dX the gradient of the
// smeared stream,
//   de_t = dX_t + gate_{t+1} dX_{t+1} + [c < 24] dz_t w_c,
//   dgate_t = dX_t . e_{t-1},  dz_t = dgate_t lam s_t (1 - s_t).
// dX = g (+ g0: the gradient reaching x0 through the residual scalars).
// Partials per workgroup: [0] sum dgate_t s_t (d lam), [1 + c] sum dz_t e_t[c] (d w).
__global__ void __launch_bounds__(256) smear_bwd_kernel(const int* __restrict__ ids, const uint16_t* __restrict__ wte,
                                                        const uint16_t* __restrict__ sw, const uint16_t* __restrict__ slam,
                                                        const float* __restrict__ g, const float* __restrict__ g0,
                                                        const float* __restrict__ sig, float* __restrict__ de,
                                                        float* __restrict__ part, int B, int T, int d, int V) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long N = (long long)B * T;
  // slam NULL: no smear, de = g + g0 only
  const float lam = slam ? bfv(slam) : 0.f;
  float acc = 0.f;  // lane c < 24: d w_c; lane 24: d lam
  for (long long n = (long long)blockIdx.x * 4 + wave; n < N; n += (long long)gridDim.x * 4) {
    const int b = (int)(n / T), t = (int)(n % T);
    const long long row = (long long)b * (T + 1) + t;
    const int id = ids[row];
    const bool ok = id >= 0 && id < V;
    const uint16_t* e = wte + (long long)(ok ? id : 0) * d;
    const int idp = t > 0 ? ids[row - 1] : -1;
    // an out-of-range previous token was gathered as a zero row: nothing to smear
    const bool has_prev = t > 0 && idp >= 0 && idp < V, has_next = t + 1 < T;
    const uint16_t* ep = has_prev ? wte + (long long)idp * d : e;
    const float st = sig[n];
    const float gnext = has_next ? lam * sig[n + 1] : 0.f;
    const float* gr = g + n * d;
    const float* g0r = g0 ? g0 + n * d : nullptr;
    const long long nn = has_next ? n + 1 : n;
    float dot = 0.f;
    for (int c = lane; c < d / 4; c += 64) {
      float4 v = *reinterpret_cast<const float4*>(gr + c * 4);
      if (g0r) {
        const float4 u = *reinterpret_cast<const float4*>(g0r + c * 4);
        v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
      }
      const uint2 p = *reinterpret_cast<const uint2*>(ep + c * 4);
      dot += v.x * lo_bf(p.x) + v.y * hi_bf(p.x) + v.z * lo_bf(p.y) + v.w * hi_bf(p.y);
    }
    dot = has_prev ? wave_sum(dot) : 0.f;
    const float dz = dot * lam * st * (1.f - st);
    float* der = de + n * d;
    for (int c = lane; c < d / 4; c += 64) {
      float4 v = *reinterpret_cast<const float4*>(gr + c * 4);
      float4 vn = *reinterpret_cast<const float4*>(g + nn * d + c * 4);
      if (g0r) {
        const float4 u = *reinterpret_cast<const float4*>(g0r + c * 4);
        const float4 un = *reinterpret_cast<const float4*>(g0 + nn * d + c * 4);
        v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
        vn.x += un.x; vn.y += un.y; vn.z += un.z; vn.w += un.w;
      }
      v.x += gnext * vn.x; v.y += gnext * vn.y; v.z += gnext * vn.z; v.w += gnext * vn.w;
      if (slam && c < kSmearCh / 4) {  // the gate's input channels also receive dz w
        v.x += dz * bfv(sw + 4 * c); v.y += dz * bfv(sw + 4 * c + 1);
        v.z += dz * bfv(sw + 4 * c + 2); v.w += dz * bfv(sw + 4 * c + 3);
      }
      *reinterpret_cast<float4*>(der + c * 4) = v;
    }
    if (lane < kSmearCh && ok) acc += dz * bfv(e + lane);
    if (lane == kSmearCh) acc += dot * st;
  }
  __shared__ float red[4][kSmearCh + 1];
  if (lane <= kSmearCh) red[wave][lane] = acc;
  __syncthreads();
  if (threadIdx.x <= kSmearCh) {
    const int v = threadIdx.x;
    const float s = red[0][v] + red[1][v] + red[2][v] + red[3][v];
    // slot 0: d lam, slots 1..24: d w
    part[(long long)blockIdx.x * (kSmearCh + 1) + (v == kSmearCh ? 0 : v + 1)] = s;
  }
}

// ---------------------------------------------------------------------------
// x <- a x + b y, then RMSNorm of the new x (one wave per row).  a = *pa (1
// when NULL), b = bsign * *pb (bf16 scalars).  xin (nullable) keeps bf16(x)
// from before the mix.
// ---------------------------------------------------------------------------
template <int MC>  // float4 chunks per lane, ceil(d / 256)
__global__ void __launch_bounds__(256) mix_rmsnorm_fwd_kernel(float* __restrict__ x, const float* __restrict__ y,
                                                              const uint16_t* __restrict__ pa,
                                                              const uint16_t* __restrict__ pb, float bsign,
                                                              uint16_t* __restrict__ xin, uint16_t* __restrict__ h,
                                                              float* __restrict__ r, long long N, int d,
                                                              float* __restrict__ amax_part) {
  const int lane = threadIdx.x & 63;
  const long long n = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int nc = d / 4;
  const float a = pa ? bfv(pa) : 1.f, bb = bsign * bfv(pb);
  float* xr = x + n * d;
  const float* yr = y + n * d;
  float4 v[MC];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int c = i * 64 + lane;
    if (c < nc) {
      const float4 xv = *reinterpret_cast<const float4*>(xr + c * 4);
      const float4 yv = *reinterpret_cast<const float4*>(yr + c * 4);
      if (xin)
        *reinterpret_cast<uint2*>(xin + n * d + c * 4) = make_uint2(pack_bf2(xv.x, xv.y), pack_bf2(xv.z, xv.w));
      v[i] = make_float4(a * xv.x + bb * yv.x, a * xv.y + bb * yv.y, a * xv.z + bb * yv.z, a * xv.w + bb * yv.w);
      *reinterpret_cast<float4*>(xr + c * 4) = v[i];
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
  if (amax_part) {
    amx = wave_max(amx);
    if (lane == 0) amax_part[n] = amx;
  }
  if (lane == 0) r[n] = rr;
}

// ---------------------------------------------------------------------------
// value embeddings: gate_h = 3 sigmoid(h[:32] . Wg[h]); v[:, h] += gate_h VE[id][h]
// one wave per token; heads in groups of 4 (16 lanes x 8 values per head)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) ve_fwd_kernel(const int* __restrict__ ids, const uint16_t* __restrict__ h1,
                                                     int d, const uint16_t* __restrict__ wg,
                                                     const uint16_t* __restrict__ ve, uint16_t* __restrict__ v,
                                                     long long ldv, float* __restrict__ gate_out, int B, int T,
                                                     int Hkv, int V) {
  const int lane = threadIdx.x & 63;
  const long long n = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= (long long)B * T) return;
  const int b = (int)(n / T), t = (int)(n % T);
  const long long id = ids[(long long)b * (T + 1) + t];
  const float hc = lane < kVeCh ? bfv(h1 + n * d + lane) : 0.f;
  const int dkv = Hkv * 128;
  for (int h0 = 0; h0 < Hkv; h0 += 4) {  // wave-uniform
    float g4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = h0 + j;
      float p = (lane < kVeCh && hh < Hkv) ? hc * bfv(wg + hh * kVeCh + lane) : 0.f;
      p = wave_sum(p);
      g4[j] = 3.f * sigm(p);
    }
    const int j = lane >> 4, hh = h0 + j;
    if (hh < Hkv) {
      const float gh = j == 0 ? g4[0] : j == 1 ? g4[1] : j == 2 ? g4[2] : g4[3];
      const int e0 = hh * 128 + (lane & 15) * 8;
      const uint4 q = (id >= 0 && id < V) ? *reinterpret_cast<const uint4*>(ve + id * dkv + e0)
                                          : make_uint4(0u, 0u, 0u, 0u);
      uint4* vp = reinterpret_cast<uint4*>(v + n * ldv + e0);
      const uint4 a = *vp;
      *vp = make_uint4(pack_bf2(lo_bf(a.x) + gh * lo_bf(q.x), hi_bf(a.x) + gh * hi_bf(q.x)),
                       pack_bf2(lo_bf(a.y) + gh * lo_bf(q.y), hi_bf(a.y) + gh * hi_bf(q.y)),
                       pack_bf2(lo_bf(a.z) + gh * lo_bf(q.z), hi_bf(a.z) + gh * hi_bf(q.z)),
                       pack_bf2(lo_bf(a.w) + gh * lo_bf(q.w), hi_bf(a.w) + gh * hi_bf(q.w)));
      if ((lane & 15) == 0) gate_out[n * Hkv + hh] = gh;
    }
  }
}

// Per token: contrib[n][h] = gate_h dv[:, h] (fp32 [N, dkv], summed into the
// table by the embedding gather); dz_h = (dv_h . VE[id][h]) gate_h (1 - gate_h / 3)
__global__ void __launch_bounds__(256) ve_bwd_kernel(const int* __restrict__ ids, const uint16_t* __restrict__ dv,
                                                     long long lddv, const uint16_t* __restrict__ ve,
                                                     const float* __restrict__ gate, float* __restrict__ contrib,
                                                     float* __restrict__ dz, int B, int T, int Hkv, int V) {
  const int lane = threadIdx.x & 63;
  const long long n = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= (long long)B * T) return;
  const int b = (int)(n / T), t = (int)(n % T);
  const long long id = ids[(long long)b * (T + 1) + t];
  const int dkv = Hkv * 128;
  for (int h0 = 0; h0 < Hkv; h0 += 4) {  // wave-uniform
    const int hh = h0 + (lane >> 4);
    const bool ok = hh < Hkv;
    const int e0 = hh * 128 + (lane & 15) * 8;
    float dvv[8], vev[8];
    float dot = 0.f;
    if (ok) {
      const uint4 a = *reinterpret_cast<const uint4*>(dv + n * lddv + e0);
      const uint4 q = (id >= 0 && id < V) ? *reinterpret_cast<const uint4*>(ve + id * dkv + e0)
                                          : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dvv[2 * k] = lo_bf(aw[k]); dvv[2 * k + 1] = hi_bf(aw[k]);
        vev[2 * k] = lo_bf(qw[k]); vev[2 * k + 1] = hi_bf(qw[k]);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) dot += dvv[k] * vev[k];
    }
    // sum over the 16 lanes of this head
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 64);
    if (ok) {
      const float gh = gate[n * Hkv + hh];
      if ((lane & 15) == 0) dz[n * Hkv + hh] = dot * gh * (1.f - gh * (1.f / 3.f));
      float* dst = contrib + n * dkv + e0;
      *reinterpret_cast<float4*>(dst) = make_float4(gh * dvv[0], gh * dvv[1], gh * dvv[2], gh * dvv[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(gh * dvv[4], gh * dvv[5], gh * dvv[6], gh * dvv[7]);
    }
  }
}

// partial sums of dWg[h][c] = sum_n dz[n, h] h1[n, c] (c < 32) over a token range per workgroup
__global__ void __launch_bounds__(256) ve_gate_grad_kernel(const float* __restrict__ dz, const uint16_t* __restrict__ h1,
                                                           int d, long long N, int Hkv, float* __restrict__ part) {
  const int np = Hkv * kVeCh;
  const long long per = (N + gridDim.x - 1) / gridDim.x;
  const long long n0 = (long long)blockIdx.x * per, n1 = min(N, n0 + per);
  for (int p = threadIdx.x; p < np; p += 256) {
    const int hh = p / kVeCh, c = p % kVeCh;
    float acc = 0.f;
    for (long long n = n0; n < n1; ++n) acc += dz[n * Hkv + hh] * bfv(h1 + n * d + c);
    part[(long long)blockIdx.x * np + p] = acc;
  }
}

// dh[n, c] = bf16(dh[n, c] + bf16(sum_h dz[n, h] Wg[h][c]))  (c < 32): the gate's
// share of the gradient of h1 joins the q/k/v product's in the same bf16 tensor
__global__ void __launch_bounds__(256) ve_dh_kernel(const float* __restrict__ dz, const uint16_t* __restrict__ wg,
                                                    uint16_t* __restrict__ dh, int d, long long N, int Hkv) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= N * kVeCh) return;
  const long long n = i / kVeCh;
  const int c = (int)(i % kVeCh);
  float acc = 0.f;
  for (int hh = 0; hh < Hkv; ++hh) acc += dz[n * Hkv + hh] * bfv(wg + hh * kVeCh + c);
  dh[n * d + c] = f2bf(bf2f(dh[n * d + c]) + bf2f(f2bf(acc)));
}

// ---------------------------------------------------------------------------
// residual scaling backward: x' = a x_in + b x0 with g = dL/dx':
//   partial sums of g . x_in and g . x0; g0 (+)= b g; g <- a g; g_bf = bf16(g)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) resid_bwd_kernel(float* __restrict__ g, uint16_t* __restrict__ g_bf,
                                                        const uint16_t* __restrict__ xin, const float* __restrict__ x0,
                                                        float* __restrict__ g0, int g0_first,
                                                        const uint16_t* __restrict__ pa,
                                                        const uint16_t* __restrict__ pb, long long n4,
                                                        float* __restrict__ part) {
  const float a = bfv(pa), bb = bfv(pb);
  float s_in = 0.f, s_0 = 0.f;
  // two chunks per thread and iteration, every load of both issued before
  // the stores (one chunk at a time left the streams' loads waiting behind
  // the previous chunk's stores)
  const long long stride = (long long)gridDim.x * 256;
  for (long long i0 = (long long)blockIdx.x * 256 + threadIdx.x; i0 < n4; i0 += 2 * stride) {
    float4 gv[2], zv[2], o[2];
    uint2 xw[2];
    bool ok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const long long i = i0 + u * stride;
      ok[u] = i < n4;
      const long long j = ok[u] ? i : i0;
      gv[u] = reinterpret_cast<const float4*>(g)[j];
      xw[u] = reinterpret_cast<const uint2*>(xin)[j];
      zv[u] = reinterpret_cast<const float4*>(x0)[j];
      o[u] = g0_first ? make_float4(0.f, 0.f, 0.f, 0.f) : reinterpret_cast<const float4*>(g0)[j];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!ok[u]) continue;
      const long long i = i0 + u * stride;
      float4 gg = gv[u];
      s_in += gg.x * lo_bf(xw[u].x) + gg.y * hi_bf(xw[u].x) + gg.z * lo_bf(xw[u].y) + gg.w * hi_bf(xw[u].y);
      s_0 += gg.x * zv[u].x + gg.y * zv[u].y + gg.z * zv[u].z + gg.w * zv[u].w;
      float4 oo = o[u];
      oo.x += bb * gg.x; oo.y += bb * gg.y; oo.z += bb * gg.z; oo.w += bb * gg.w;
      reinterpret_cast<float4*>(g0)[i] = oo;
      gg.x *= a; gg.y *= a; gg.z *= a; gg.w *= a;
      reinterpret_cast<float4*>(g)[i] = gg;
      reinterpret_cast<uint2*>(g_bf)[i] = make_uint2(pack_bf2(gg.x, gg.y), pack_bf2(gg.z, gg.w));
    }
  }
  s_in = wave_sum(s_in);
  s_0 = wave_sum(s_0);
  __shared__ float red[2][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { red[0][wave] = s_in; red[1][wave] = s_0; }
  __syncthreads();
  if (threadIdx.x < 2)
    part[(long long)blockIdx.x * 2 + threadIdx.x] =
        red[threadIdx.x][0] + red[threadIdx.x][1] + red[threadIdx.x][2] + red[threadIdx.x][3];
}

// backout backward at the head: partial sums of g . x_mid, and a copy of g
__global__ void __launch_bounds__(256) backout_bwd_kernel(const float* __restrict__ g, const float* __restrict__ xm,
                                                          float* __restrict__ gcopy, long long n4,
                                                          float* __restrict__ part) {
  float s = 0.f;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
    const float4 gv = reinterpret_cast<const float4*>(g)[i];
    const float4 xv = reinterpret_cast<const float4*>(xm)[i];
    s += gv.x * xv.x + gv.y * xv.y + gv.z * xv.z + gv.w * xv.w;
    reinterpret_cast<float4*>(gcopy)[i] = gv;
  }
  s = wave_sum(s);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// g += c y with c = csign * *pc (bf16 scalar); g_bf = bf16(g)
__global__ void __launch_bounds__(256) axpy_stream_kernel(float* __restrict__ g, uint16_t* __restrict__ g_bf,
                                                          const float* __restrict__ y, const uint16_t* __restrict__ pc,
                                                          float csign, long long n4) {
  const float c = csign * bfv(pc);
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
    float4 gv = reinterpret_cast<const float4*>(g)[i];
    const float4 yv = reinterpret_cast<const float4*>(y)[i];
    gv.x += c * yv.x; gv.y += c * yv.y; gv.z += c * yv.z; gv.w += c * yv.w;
    reinterpret_cast<float4*>(g)[i] = gv;
    reinterpret_cast<uint2*>(g_bf)[i] = make_uint2(pack_bf2(gv.x, gv.y), pack_bf2(gv.z, gv.w));
  }
}

// out[v] = beta out[v] + scale sum_p part[p nvals + v]
// Value v = sum over p < nparts of part[p * nvals + v], one workgroup per
// value: fixed per-thread strides, then a fixed tree in LDS, in double (a
// thread per value summing the partials one after another took about 150 us
// per reduction, each load waited for).  Values v < nlo go to out_lo[v], the
// others to out_hi[v - nlo] (two parameter slots in one launch);
// out = beta out + scale sum.
__global__ void __launch_bounds__(256) reduce_partials_kernel(const float* __restrict__ part, int nparts, int nvals,
                                                              float* __restrict__ out_lo, int nlo,
                                                              float* __restrict__ out_hi, float scale, float beta) {
  const int v = blockIdx.x;
  double s = 0.0;
  for (int p = threadIdx.x; p < nparts; p += 256) s += part[(long long)p * nvals + v];
  __shared__ double red[256];
  red[threadIdx.x] = s;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float* o = v < nlo ? out_lo + v : out_hi + (v - nlo);
    const float r = scale * (float)red[0];
    *o = beta != 0.f ? beta * *o + r : r;
  }
}

}  // namespace

constexpr int kFeatBlocks = 1024;  // workgroups of the grid-stride reductions

long long feature_partial_floats(int Hkv) {
  // partial rows of the largest reduction, plus room for the reduced totals
  return std::max<long long>(std::max<long long>((long long)kFeatBlocks * 2, (long long)kFeatBlocks * (kSmearCh + 1)),
                             (long long)kFeatBlocks * Hkv * kVeCh) + 64;
}

// values [0, nlo) into out_lo, [nlo, nvals) into out_hi
static int reduce_to2(const float* part, int nparts, int nvals, float* out_lo, int nlo, float* out_hi, float scale,
                      bool accumulate, hipStream_t s) {
  hipLaunchKernelGGL(reduce_partials_kernel, dim3(nvals), dim3(256), 0, s, part, nparts, nvals, out_lo, nlo, out_hi,
                     scale, accumulate ? 1.f : 0.f);
  GS_LAUNCH_CHECK("reduce_partials");
  return 0;
}

static int reduce_to(const float* part, int nparts, int nvals, float* out, float scale, bool accumulate,
                     hipStream_t s) {
  return reduce_to2(part, nparts, nvals, out, nvals, nullptr, scale, accumulate, s);
}

int launch_smear_fwd(const int* ids, const uint16_t* wte, const uint16_t* sw, const uint16_t* slam, float* x,
                     float* x0, float* sig, int B, int T, int d, int V, hipStream_t s) {
  hipLaunchKernelGGL(smear_fwd_kernel, dim3(nblocks((long long)B * T, 4)), dim3(256), 0, s, ids, wte, sw, slam, x, x0,
                     sig, B, T, d, V);
  GS_LAUNCH_CHECK("smear_fwd");
  return 0;
}

int launch_smear_bwd(const int* ids, const uint16_t* wte, const uint16_t* sw, const uint16_t* slam, const float* g,
                     const float* g0, const float* sig, float* de, float* part, float* dlam, float* dw,
                     bool accumulate, int B, int T, int d, int V, hipStream_t s) {
  hipLaunchKernelGGL(smear_bwd_kernel, dim3(kFeatBlocks), dim3(256), 0, s, ids, wte, sw, slam, g, g0, sig, de, part,
                     B, T, d, V);
  GS_LAUNCH_CHECK("smear_bwd");
  if (!slam) return 0;
  // part rows: [d lam, d w_0 .. d w_23]; d lam and d w are separate parameter slots
  return reduce_to2(part, kFeatBlocks, kSmearCh + 1, dlam, 1, dw, 1.f, accumulate, s);
}

int launch_mix_rmsnorm_fwd(float* x, const float* y, const uint16_t* pa, const uint16_t* pb, float bsign,
                           uint16_t* xin, uint16_t* h, float* r, long long N, int d, float* amax_part, hipStream_t s) {
  const int mc = (d / 4 + 63) / 64;
#define GS_MR(M)                                                                                                     \
  hipLaunchKernelGGL((mix_rmsnorm_fwd_kernel<M>), dim3(nblocks(N, 4)), dim3(256), 0, s, x, y, pa, pb, bsign, xin, h, \
                     r, N, d, amax_part)
  switch (mc) {
    case 1: GS_MR(1); break;
    case 2: GS_MR(2); break;
    case 3: GS_MR(3); break;
    case 4: GS_MR(4); break;
    case 5: GS_MR(5); break;
    case 6: GS_MR(6); break;
    case 7: GS_MR(7); break;
    case 8: GS_MR(8); break;
    default: GS_MR(kMaxChunks); break;
  }
#undef GS_MR
  GS_LAUNCH_CHECK("mix_rmsnorm_fwd");
  return 0;
}

int launch_ve_fwd(const int* ids, const uint16_t* h1, int d, const uint16_t* wg, const uint16_t* ve, uint16_t* v,
                  long long ldv, float* gate, int B, int T, int Hkv, int V, hipStream_t s) {
  hipLaunchKernelGGL(ve_fwd_kernel, dim3(nblocks((long long)B * T, 4)), dim3(256), 0, s, ids, h1, d, wg, ve, v, ldv,
                     gate, B, T, Hkv, V);
  GS_LAUNCH_CHECK("ve_fwd");
  return 0;
}

int launch_ve_bwd(const int* ids, const uint16_t* dv, long long lddv, const uint16_t* ve, const float* gate,
                  float* contrib, float* dz, int B, int T, int Hkv, int V, hipStream_t s) {
  hipLaunchKernelGGL(ve_bwd_kernel, dim3(nblocks((long long)B * T, 4)), dim3(256), 0, s, ids, dv, lddv, ve, gate,
                     contrib, dz, B, T, Hkv, V);
  GS_LAUNCH_CHECK("ve_bwd");
  return 0;
}

int launch_ve_gate_grad(const float* dz, const uint16_t* h1, int d, long long N, int Hkv, float* part, float* dwg,
                        bool accumulate, hipStream_t s) {
  hipLaunchKernelGGL(ve_gate_grad_kernel, dim3(kFeatBlocks), dim3(256), 0, s, dz, h1, d, N, Hkv, part);
  GS_LAUNCH_CHECK("ve_gate_grad");
  return reduce_to(part, kFeatBlocks, Hkv * kVeCh, dwg, 1.f, accumulate, s);
}

int launch_ve_dh(const float* dz, const uint16_t* wg, uint16_t* dh, int d, long long N, int Hkv, hipStream_t s) {
  hipLaunchKernelGGL(ve_dh_kernel, dim3(nblocks(N * kVeCh, 256)), dim3(256), 0, s, dz, wg, dh, d, N, Hkv);
  GS_LAUNCH_CHECK("ve_dh");
  return 0;
}

int launch_resid_bwd(float* g, uint16_t* g_bf, const uint16_t* xin, const float* x0, float* g0, bool g0_first,
                     const uint16_t* pa, const uint16_t* pb, long long n, float* part, float* da, float* db,
                     bool accumulate, hipStream_t s) {
  hipLaunchKernelGGL(resid_bwd_kernel, dim3(kFeatBlocks), dim3(256), 0, s, g, g_bf, xin, x0, g0, (int)g0_first, pa, pb,
                     n / 4, part);
  GS_LAUNCH_CHECK("resid_bwd");
  // part rows: [g . x_in, g . x0] into the two scalars' slots
  return reduce_to2(part, kFeatBlocks, 2, da, 1, db, 1.f, accumulate, s);
}

int launch_backout_bwd(const float* g, const float* xm, float* gcopy, long long n, float* part, float* dlam,
                       bool accumulate, hipStream_t s) {
  hipLaunchKernelGGL(backout_bwd_kernel, dim3(kFeatBlocks), dim3(256), 0, s, g, xm, gcopy, n / 4, part);
  GS_LAUNCH_CHECK("backout_bwd");
  // x_final = x - lam x_mid: d lam = -sum g . x_mid
  return reduce_to(part, kFeatBlocks, 1, dlam, -1.f, accumulate, s);
}

int launch_axpy_stream(float* g, uint16_t* g_bf, const float* y, const uint16_t* pc, float csign, long long n,
                       hipStream_t s) {
  hipLaunchKernelGGL(axpy_stream_kernel, dim3(kFeatBlocks), dim3(256), 0, s, g, g_bf, y, pc, csign, n / 4);
  GS_LAUNCH_CHECK("axpy_stream");
  return 0;
}

}  // namespace gs
