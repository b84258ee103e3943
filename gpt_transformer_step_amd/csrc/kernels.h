// Internal launchers of the non-GEMM kernels of libgptstep.  All take device
// pointers, enqueue on `s` and return 0 or a gpt_status error code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gs {

// --- elementwise / bandwidth-bound (elementwise.hip) -----------------------
int launch_fill_f32(float* p, long long n, float v, hipStream_t s);
int launch_cast_bf16(const float* src, uint16_t* dst, long long n, hipStream_t s);
int launch_rope_table(float* cos_sin /* [T, 64] cos then [T, 64] sin */, int T, hipStream_t s);
int launch_embed_fwd(const int* ids, const uint16_t* wte, float* x, int B, int T, int d, int V, hipStream_t s);
// scratch bytes of the embedding backward's sort (rows of T + 1 ids per
// sequence; ids outside [0, V) take no part)
size_t embed_bwd_workspace(long long N, int V);
// stable counting sort of the token ids (ws: embed_bwd_workspace bytes), then
// dst[v] (+)= sum over the tokens of id v, in token order, of g [N, d] rows
// (d % 4 == 0); the gather may run several times on one sort
int launch_embed_sort(const int* ids, int B, int T, int V, void* ws, hipStream_t s);
int launch_embed_gather(const float* g, float* dst, long long N, int d, int V, bool accumulate, const void* ws,
                        hipStream_t s);
// amax_part (nullable): per-row max |stored bf16 value| at amax_part[row]
int launch_rmsnorm_fwd(const float* x, uint16_t* h, float* r, long long N, int d, hipStream_t s,
                       float* amax_part = nullptr);
// dh: bf16 (dh_bf16) or fp32, rounded to bf16 as it is read
int launch_rmsnorm_bwd(const void* dh, bool dh_bf16, const uint16_t* h, const float* r, float* g, uint16_t* g_bf,
                       long long N, int d, hipStream_t s, float* amax_part = nullptr);
// dz [N, ld] bf16 = scale (softmax - onehot(target)) on the nv vocabulary
// columns c0 .. c0+nv-1, from the fp16 exponentials e [N, ld] = exp(z - mx)
// the cross-entropy forward kept, mx from its (max, sum) partials [N, nparts]
// of cw columns each
int launch_ce_dz(const uint16_t* e, uint16_t* dz, const float* part, int nparts, int cw, int c0, const float* lse,
                 const int* ids, int T, long long N, int nv, int ld, float scale, hipStream_t s);
int launch_ce_reduce(const float* part, int nparts, const float* zt, float* lse, float* row_loss,
                     float* lse_out, long long N, hipStream_t s);
int launch_loss_mean(const float* row_loss, float* loss, long long N, hipStream_t s);
// C[b][i][j] = C[b][j][i] for i > j (bf16 n x n matrices, row stride ld, batch stride stride)
int launch_sym_mirror(uint16_t* C, int n, long long ld, long long stride, int count, hipStream_t s);
// out[0..n) = beta * out + sum_{s < nsplit} part[s * stride + i]; optional bf16 copy out_bf;
// out nullable (then beta 0 and out_bf given)
int launch_splitk_reduce(const float* part, int nsplit, long long stride, float* out, uint16_t* out_bf, long long n,
                         float beta, hipStream_t s);

// --- Muon elementwise (elementwise.hip) ------------------------------------
// M <- mu M + G (count matrices of per elements, 16-byte aligned) and the
// Frobenius partial sums of the new M, as launch_frob_partial writes them
int launch_momentum_frob(float* M, const float* G, float mu, float* partial, int count, long long per, int nblk,
                         hipStream_t s);
int launch_frob_partial(const float* X, float* partial, int count, long long per, int nblk,
                        hipStream_t s);
// X[b] (oriented [l, s]) = src[b] / (||src[b]|| + eps); transposed when rows < cols
int launch_ns_init(const float* src, const float* partial, int nblk, float* X, uint16_t* Xb,
                   int count, int rows, int cols, float eps, hipStream_t s);
// O = X (bf16) oriented back (times the NorMuon scale nsc of its row (nm_rows)
// or column when nsc is given); W = W (1 - lr wd) - lr O; W_bf16 = bf16(W); O_out = O
int launch_muon_apply(const uint16_t* X, float* W, uint16_t* Wb, float* O_out, int count, int rows,
                      int cols, float lr, float wd, const float* nsc, int nm_rows, hipStream_t s);
// NorMuon: from the orthogonalised X (oriented as for launch_muon_apply),
// update the per-neuron second moments V and write the per-neuron scale
// (neurons = rows of W when per_row, else columns); part: scratch of
// normuon_part_floats floats
int launch_normuon_scale(const uint16_t* X, float* part, float* V, float* scale, int count, int rows, int cols,
                         int per_row, float beta2, float eps, hipStream_t s);
long long normuon_part_floats(int count, int rows, int cols);

// AdamW on n fp32 parameters (n % 4 == 0, 16-byte aligned; Wb nullable)
int launch_adamw(float* W, uint16_t* Wb, const float* G, float* M, float* V, long long n, float lr, float b1,
                 float b2, float eps, float wd, float inv_bc1, float inv_bc2, float gs, hipStream_t s);

// --- record-model features (features.hip) ----------------------------------
// scalars (pa, pb, pc, slam) and small weights are device bf16 values
// scratch floats of the partial-sum reductions below
long long feature_partial_floats(int Hkv);
// x = e_t + lam sigmoid(e_t[:24] . sw) e_{t-1} (token 0: e_0); x0 (nullable) = copy; sig = the sigmoids
int launch_smear_fwd(const int* ids, const uint16_t* wte, const uint16_t* sw, const uint16_t* slam, float* x,
                     float* x0, float* sig, int B, int T, int d, int V, hipStream_t s);
// de = backward of smear for dX = g (+ g0); d lam and d sw written (or added) to dlam / dw
int launch_smear_bwd(const int* ids, const uint16_t* wte, const uint16_t* sw, const uint16_t* slam, const float* g,
                     const float* g0, const float* sig, float* de, float* part, float* dlam, float* dw,
                     bool accumulate, int B, int T, int d, int V, hipStream_t s);
// x <- a x + bsign b y (a = 1 when pa is NULL); xin (nullable) = bf16(old x); h, r = RMSNorm of new x
int launch_mix_rmsnorm_fwd(float* x, const float* y, const uint16_t* pa, const uint16_t* pb, float bsign,
                           uint16_t* xin, uint16_t* h, float* r, long long N, int d, float* amax_part, hipStream_t s);
// v[:, head] += 3 sigmoid(h1[:32] . wg[head]) ve[id][head]; gate [N, Hkv] saved
int launch_ve_fwd(const int* ids, const uint16_t* h1, int d, const uint16_t* wg, const uint16_t* ve, uint16_t* v,
                  long long ldv, float* gate, int B, int T, int Hkv, int V, hipStream_t s);
// contrib [N, dkv] fp32 = gate dv per token (the table gradient is its sum per
// id, by launch_embed_gather); dz = (dv . ve) gate (1 - gate / 3)
int launch_ve_bwd(const int* ids, const uint16_t* dv, long long lddv, const uint16_t* ve, const float* gate,
                  float* contrib, float* dz, int B, int T, int Hkv, int V, hipStream_t s);
// dwg (+)= dz^T h1[:, :32]
int launch_ve_gate_grad(const float* dz, const uint16_t* h1, int d, long long N, int Hkv, float* part, float* dwg,
                        bool accumulate, hipStream_t s);
// dh[:, :32] = bf16(dh[:, :32] + bf16(dz wg)), dh bf16
int launch_ve_dh(const float* dz, const uint16_t* wg, uint16_t* dh, int d, long long N, int Hkv, hipStream_t s);
// backward of x' = a x_in + b x0: da, db (+)= g.x_in, g.x0; g0 (first: =) += b g; g = a g; g_bf
int launch_resid_bwd(float* g, uint16_t* g_bf, const uint16_t* xin, const float* x0, float* g0, bool g0_first,
                     const uint16_t* pa, const uint16_t* pb, long long n, float* part, float* da, float* db,
                     bool accumulate, hipStream_t s);
// backout at the head: dlam (+)= -g . x_mid; gcopy = g
int launch_backout_bwd(const float* g, const float* xm, float* gcopy, long long n, float* part, float* dlam,
                       bool accumulate, hipStream_t s);
// g += csign c y; g_bf = bf16(g)
int launch_axpy_stream(float* g, uint16_t* g_bf, const float* y, const uint16_t* pc, float csign, long long n,
                       hipStream_t s);

// --- attention (attention.hip) ---------------------------------------------
// H query heads, Hkv key/value heads (query head h reads head h / (H / Hkv));
// window: left window (query i sees keys i - window .. i), -1 = full causal
// lse [B, H, T]: natural log-sum-exp of each row's scaled scores, or (lse_log2)
// in log2 units, the form the fused backward kernels (QkNormBwd given) read
// amax (nullable): per-wave max |stored output| (attn_fwd_amax_slots of them)
int launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, long long ld_qkv,
                    uint16_t* out, long long ld_out, float* lse, int B, int H, int Hkv, int T, int window,
                    hipStream_t s, bool lse_log2 = false, float* amax = nullptr);
long long attn_fwd_amax_slots(int B, int H, int T);
long long attn_bwd_amax_slots(int B, int H, int Hkv, int T);
int launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, long long ld_qkv,
                    const uint16_t* out, const uint16_t* dout, long long ld_out, const float* lse,
                    float* delta, float* dq, uint16_t* dk, uint16_t* dv, long long ld_dkv, int B,
                    int H, int Hkv, int T, int window, hipStream_t s);
// The QK-norm + rotary backward fused into the attention backward: q and k
// are the stored normed, rotated heads; rq [N, H] and rk [N, Hkv] their
// inverse RMS; cs the rotary table; dq (bf16, row stride ld_dkv) receives the
// gradient of the raw query heads, dk that of the raw key heads.
struct QkNormBwd {
  const float* rq;
  const float* rk;
  const float* cs;
  uint16_t* dq;
  float* amax;  // nullable: per-wave max |stored dq, dk, dv| (attn_bwd_amax_slots of them)
};
// one of the two backward kernels, in this order: 0 = dQ (also writes -rowsum(dout * out) into
// delta), 1 = dK/dV (reads it).  fuse NULL: raw gradients (dq fp32 [N, 128 H], dk bf16), lse in
// natural units; else the gradients of the raw heads through the QK-norm and rotary
// backward, lse in log2 units.
int launch_attn_bwd_part(int part, const uint16_t* q, const uint16_t* k, const uint16_t* v, long long ld_qkv,
                         const uint16_t* out, const uint16_t* dout, long long ld_out, const float* lse, float* delta,
                         float* dq, uint16_t* dk, uint16_t* dv, long long ld_dkv, int B, int H, int Hkv, int T,
                         int window, hipStream_t s, const QkNormBwd* fuse);

// --- fp8 quantisation (fp8.hip) --------------------------------------------
// Tensors are [rows, cols] with row stride ld (elements); rows % 16 == 0,
// cols % 16 == 0, rows * cols / 4 < 2^31.  fmt 0 = E4M3, 1 = E5M2.
constexpr int kFp8Partials = 1024;  // floats of `partial` scratch per tensor
int fp8_partials(long long rows, long long cols);
// scale[0] = fmax / max|x| (1 when x == 0).  Batched: count tensors of one
// shape, tensor b at x + b sx (elements), its scale at scale[b sscale]; the
// partials need count * fp8_partials(rows, cols) floats.
int launch_fp8_amax_scale(const void* x, int is_f32, long long ldx, int rows, int cols, int fmt, float* partial,
                          float* scale, hipStream_t s, int count = 1, long long sx = 0, long long sscale = 0);
// q[r, c] = code(x[r, c] * scale) and / or qt[c, r] = the same code (each nullable);
// batched as above, tensor b's codes at q + b sq and qt + b sq
int launch_fp8_quant(const void* x, int is_f32, long long ldx, int rows, int cols, int fmt, const float* scale,
                     uint8_t* q, long long ldq, uint8_t* qt, long long ldqt, hipStream_t s, int count = 1,
                     long long sx = 0, long long sscale = 0, long long sq = 0);
int quantize_fp8(const void* x, int is_f32, long long ldx, int rows, int cols, int fmt, float* partial, float* scale,
                 uint8_t* q, long long ldq, uint8_t* qt, long long ldqt, hipStream_t s);
// the same with the amax already reduced by the producer into np partials
int quantize_fp8_partials(const void* x, int is_f32, long long ldx, int rows, int cols, int fmt,
                          const float* partial, long long np, float* scale, uint8_t* q, long long ldq, uint8_t* qt,
                          long long ldqt, hipStream_t s);

// --- roofline probes (probe.hip) -------------------------------------------
int launch_mfma_peak(int fp8, int blocks, int iters, float* out, double* flops, hipStream_t s);

}  // namespace gs
