/*
 * gptstep_ops.h -- component entry points of libgptstep.so.
 *
 * These expose the individual steps that gpt_step_fwd / gpt_step_bwd /
 * muon_update chain together, so each can be checked on its own.  They use
 * the same kernels as the step entry points and follow the conventions of
 * gptstep.h (device pointers unless marked host; caller-owned memory; host
 * validation first; asynchronous on `stream`; status return).
 */
#ifndef GPTSTEP_OPS_H
#define GPTSTEP_OPS_H

#include "gptstep.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Operand layouts of gpt_op_gemm.  An operand is a logical [rows, K] matrix:
 *   GPT_LAYOUT_K_CONTIG : element (r, k) at X[r * ld + k]   (row-major [rows, K])
 *   GPT_LAYOUT_MN_CONTIG: element (r, k) at X[k * ld + r]   (row-major [K, rows]) */
enum { GPT_LAYOUT_K_CONTIG = 0, GPT_LAYOUT_MN_CONTIG = 1 };
enum { GPT_DTYPE_F32 = 0, GPT_DTYPE_BF16 = 1 };

/* Batched bf16 matrix product with fp32 accumulation (the linear layers of
 * dev.to "¿Cómo Entrenar Tu Propio ChatGPT por $50?", "3. Gestión de
 * Precisión": F.linear with the weight cast to bf16):
 *   C[b][m, n] = alpha * sum_k A[b][m, k] * B[b][n, k]  (+ beta * C[b][m, n] for f32 C)
 * for b < batch, m < M, n < N, k < K.  A, B: bf16 bit patterns; strides
 * stride_* in elements between batch items; ld* in elements, multiples of 8;
 * A, B, C 16-byte aligned.  c_dtype: GPT_DTYPE_F32 or GPT_DTYPE_BF16 (beta
 * must be 0 for bf16).  M, N, K, batch >= 0 (0 is a no-op). */
gpt_status gpt_op_gemm(int32_t M, int32_t N, int32_t K, int32_t batch, const uint16_t* A,
                       int32_t a_layout, int64_t lda, int64_t stride_a, const uint16_t* B,
                       int32_t b_layout, int64_t ldb, int64_t stride_b, void* C, int32_t c_dtype,
                       int64_t ldc, int64_t stride_c, float alpha, float beta, gpt_stream_t stream);

/* fp8 formats (OCP): E4M3 (largest finite 448, no infinities) and E5M2
 * (largest finite 57344). */
enum { GPT_FP8_E4M3 = 0, GPT_FP8_E5M2 = 1 };

/* Per-tensor fp8 quantisation (apidog.com/pt "Gerenciamento de Precisão",
 * apidog.com/de "Präzisionsverwaltung": fp8 linear layers with one scale per
 * tensor).  x: [rows, cols] row-major with leading dimension ldx (elements),
 * bf16 (x_dtype = GPT_DTYPE_BF16) or fp32 (GPT_DTYPE_F32).
 *   scale[0] = fmax / max|x|  (fp32 division; 1 when x is all zero)
 *   code     = round-to-nearest-even(clamp(x * scale, -fmax, fmax))
 * q (nullable): codes [rows, cols] with leading dimension ldq;
 * qt (nullable): the same codes transposed, [cols, rows], leading dimension ldqt.
 * partial: device fp32 scratch of gpt_fp8_partials(rows, cols) floats.
 * Needs rows % 16 == 0, cols % 16 == 0, rows*cols < 2^33, ldx % 8 == 0,
 * ldq % 8 == 0, ldqt % 16 == 0; x and qt 16-byte aligned, q 8-byte aligned. */
int32_t gpt_fp8_partials(int32_t rows, int32_t cols);
gpt_status gpt_op_quantize_fp8(const void* x, int32_t x_dtype, int64_t ldx, int32_t rows, int32_t cols,
                               int32_t fmt, float* scale, uint8_t* q, int64_t ldq, uint8_t* qt,
                               int64_t ldqt, float* partial, gpt_stream_t stream);

/* fp8 matrix product with fp32 accumulation (the fp8 linear layers of the
 * precision passage above):
 *   C[m, n] = sum_k dec(A[m, k]) dec(B[n, k]) / (scale_a[0] * scale_b[0])  (+ beta * C[m, n])
 * A: logical codes [M, K] in format fmt_a, B: logical [N, K] in fmt_b, each
 * in one of the operand layouts above (GPT_LAYOUT_K_CONTIG: element (r, k)
 * at X[r * ld + k]; GPT_LAYOUT_MN_CONTIG: at X[k * ld + r]); C fp32 [M, N]
 * (ldc); scale_a, scale_b: device fp32 scalars (the quantisation scales of
 * the two operands).  Both k-contiguous: any format pair.  m/n-contiguous
 * operands (the codes of an output gradient and of an activation or weight
 * read as stored, for the weight and data gradients): A E5M2, B E4M3, B
 * m/n-contiguous, A either; the m/n-contiguous operand's rows (M or N) a
 * multiple of 16.  K % 16 == 0; lda, ldb >= the operand's contiguous
 * dimension and multiples of 16; ldc >= N, a multiple of 4; pointers 16-byte
 * aligned.  Other combinations return GPT_ERR_UNSUPPORTED. */
gpt_status gpt_op_gemm_fp8(int32_t M, int32_t N, int32_t K, const uint8_t* A, int32_t fmt_a, int32_t a_layout,
                           int64_t lda, const uint8_t* B, int32_t fmt_b, int32_t b_layout, int64_t ldb, float* C,
                           int64_t ldc, const float* scale_a, const float* scale_b, float beta, gpt_stream_t stream);

/* Causal multi-head attention forward with head width 128 (dev.to page,
 * "5. Unificación Flash Attention": flash_attn_func(q, k, v, causal=True,
 * window_size=...)):
 *   out[b,t,h,:] = sum_{j in W(t)} softmax_j(q[b,t,h,:] . k[b,j,g(h),:] / sqrt(128)) v[b,j,g(h),:]
 * with W(t) = {j : j <= t, and j >= t - window when window >= 0} (window < 0:
 * full causal) and g(h) = h / (n_head / n_kv_head) (n_kv_head divides
 * n_head).  q, out: bf16, element (b, t, h, e) at ptr[(b*T + t) * ld + h*128 + e];
 * k, v: the same with n_kv_head heads (ld in elements, multiple of 8).
 * lse: fp32 [B, H, T], the natural-log log-sum-exp of each row of scaled
 * scores (needed by the backward). */
gpt_status gpt_op_attention_fwd(int32_t batch, int32_t n_head, int32_t n_kv_head, int32_t seq_len, int32_t window,
                                const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_qkv,
                                uint16_t* out, int64_t ld_out, float* lse, gpt_stream_t stream);

/* Backward of gpt_op_attention_fwd given dout (same layout as out):
 *   dq_acc fp32, element (b,t,h,e) at dq_acc[(b*T+t) * H*128 + h*128 + e] (written);
 *   dk, dv bf16 in the k/v layout with leading dimension ld_dkv (written; a
 *   key/value head receives the sum over its query heads);
 *   delta: fp32 scratch [B, H, T] (receives -rowsum(dout * out)). */
gpt_status gpt_op_attention_bwd(int32_t batch, int32_t n_head, int32_t n_kv_head, int32_t seq_len, int32_t window,
                                const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_qkv,
                                const uint16_t* out, const uint16_t* dout, int64_t ld_out,
                                const float* lse, float* delta, float* dq_acc, uint16_t* dk,
                                uint16_t* dv, int64_t ld_dkv, gpt_stream_t stream);

/* Size in bytes and offset of a named activation inside the step workspace
 * after gpt_step_fwd, for inspection.  which: 0 residual x after the last
 * layer (fp32 [N,d]); 1 h1 of `layer` (bf16 [N,d], normed input of the
 * attention); 2 qkv of `layer` (bf16 [N,3d], q and k after rotation and
 * normalisation); 3 attention output of `layer` (bf16 [N,d]); 4 h2 of
 * `layer` (bf16 [N,d]); 5 relu^2 activation of `layer` (bf16 [N,4d]);
 * 6 final normed hidden state (bf16 [N,d]); 7 per-row lse (fp32 [N]);
 * 8 per-row loss (fp32 [N]); 9 per-row logit of the target token (fp32 [N]).
 * N = batch*seq_len. */
gpt_status gpt_workspace_tensor(const gpt_shape* shape, int32_t which, int32_t layer,
                                size_t* offset /* host */, size_t* bytes /* host */);

/* Kernel timing by category (instrumentation for measurement).  When the bit
 * of a category is set in `mask`, every launch of that category made by the
 * step entry points is bracketed with HIP events recorded on the launch
 * stream.  gpt_profile_read synchronises on those events and returns the
 * summed elapsed milliseconds and the number of bracketed launches since the
 * last reset.  Host-side state; not thread-safe.  Categories are numbered
 * 0 .. gpt_profile_num_categories()-1 and named by gpt_profile_category_name. */
int32_t gpt_profile_num_categories(void);
const char* gpt_profile_category_name(int32_t category);
gpt_status gpt_profile_enable(uint64_t mask);
gpt_status gpt_profile_reset(void);
gpt_status gpt_profile_read(int32_t category, double* total_ms /* host */, int32_t* launches /* host */);

/* Roofline probe: a matrix-core-only kernel (no memory traffic) with
 * `blocks` workgroups of 4 waves, each issuing iters x 8 independent MFMAs
 * (fp8 = 0: v_mfma_f32_32x32x16_bf16; fp8 = 1: the 32x32x64 E4M3 MFMA).
 * `out` (device, fp32 [blocks*256]) receives a checksum; *flops (host) the
 * FLOPs the launch performs.  Time it with events to get the sustained rate. */
gpt_status gpt_probe_mfma(int32_t fp8, int32_t blocks, int32_t iters, float* out, double* flops /* host */,
                          gpt_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GPTSTEP_OPS_H */
