// C ABI of libgptstep: argument validation, parameter/workspace layout and
// the launch sequence of the training step.  Kernels live in the .hip files.

#include <math.h>
#include <string.h>

#include <string>
#include <vector>

#include "common.h"
#include "gemm.h"
#include "gptstep.h"
#include "gptstep_ops.h"
#include "kernels.h"

namespace gs {

static thread_local std::string g_err;
void set_error(const std::string& msg) { g_err = msg; }

}  // namespace gs

using namespace gs;

#define FAIL(code, msg)        \
  do {                         \
    gs::set_error(msg);        \
    return (gpt_status)(code); \
  } while (0)

#define TRY(expr)                          \
  do {                                     \
    int rc_ = (expr);                      \
    if (rc_ != 0) return (gpt_status)rc_;  \
  } while (0)

static inline hipStream_t S(gpt_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------
// status
// ---------------------------------------------------------------------------
extern "C" const char* gpt_status_string(gpt_status s) {
  switch (s) {
    case GPT_OK: return "ok";
    case GPT_ERR_INVALID_ARG: return "invalid argument";
    case GPT_ERR_SHAPE: return "invalid shape";
    case GPT_ERR_WORKSPACE: return "workspace too small";
    case GPT_ERR_HIP: return "HIP runtime error";
    case GPT_ERR_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

extern "C" const char* gpt_last_error(void) { return gs::g_err.c_str(); }

extern "C" int32_t gpt_abi_version(void) { return 1; }

// ---------------------------------------------------------------------------
// shapes and layouts
// ---------------------------------------------------------------------------
namespace {

struct Dims {
  int L, d, H, hidden, V, T, B, prec;
  long long N;  // tokens per step
};

int check_shape(const gpt_shape* s, Dims* o) {
  if (!s) FAIL(GPT_ERR_INVALID_ARG, "shape is NULL");
  if (s->depth < 2 || s->depth > 64 || (s->depth & 1))
    FAIL(GPT_ERR_SHAPE, "depth must be even and in [2, 64] (heads are 128 wide, d_model = 64*depth)");
  if (s->vocab < 1 || s->vocab > (1 << 24)) FAIL(GPT_ERR_SHAPE, "vocab must be in [1, 2^24]");
  if (s->seq_len < 1 || s->seq_len > 16384) FAIL(GPT_ERR_SHAPE, "seq_len must be in [1, 16384]");
  if (s->batch < 1) FAIL(GPT_ERR_SHAPE, "batch must be >= 1");
  if ((long long)s->batch * s->seq_len > (1LL << 24)) FAIL(GPT_ERR_SHAPE, "batch*seq_len must be <= 2^24");
  if (s->precision != GPT_PREC_BF16 && s->precision != GPT_PREC_FP8)
    FAIL(GPT_ERR_UNSUPPORTED, "unknown precision");
  o->L = s->depth;
  o->d = 64 * s->depth;
  o->H = o->d / 128;
  o->hidden = 4 * o->d;
  o->V = s->vocab;
  o->T = s->seq_len;
  o->B = s->batch;
  o->prec = s->precision;
  o->N = (long long)s->batch * s->seq_len;
  return 0;
}

// element offsets of the packed parameter tensors
struct ParamLayout {
  size_t wte, lm_head, total;
  size_t qkv(const Dims& D, int l) const { return wte_end + (size_t)l * 4 * D.d * D.d; }
  size_t wo(const Dims& D, int l) const { return qkv(D, l) + (size_t)3 * D.d * D.d; }
  size_t fc(const Dims& D, int l) const { return s_end + (size_t)l * D.hidden * D.d; }
  size_t proj(const Dims& D, int l) const { return f_end + (size_t)l * D.d * D.hidden; }
  size_t wte_end, s_end, f_end, p_end;
};

ParamLayout param_layout(const Dims& D) {
  ParamLayout p;
  p.wte = 0;
  p.wte_end = (size_t)D.V * D.d;
  p.s_end = p.wte_end + (size_t)D.L * 4 * D.d * D.d;
  p.f_end = p.s_end + (size_t)D.L * D.hidden * D.d;
  p.p_end = p.f_end + (size_t)D.L * D.d * D.hidden;
  p.lm_head = p.p_end;
  p.total = p.lm_head + (size_t)D.V * D.d;
  return p;
}

}  // namespace

extern "C" gpt_status gpt_param_count(const gpt_shape* shape, size_t* n) {
  Dims D;
  TRY(check_shape(shape, &D));
  if (!n) FAIL(GPT_ERR_INVALID_ARG, "n_params is NULL");
  *n = param_layout(D).total;
  return GPT_OK;
}

extern "C" gpt_status gpt_param_layout(const gpt_shape* shape, size_t* offsets, int32_t capacity,
                                       int32_t* n_tensors) {
  Dims D;
  TRY(check_shape(shape, &D));
  if (!n_tensors) FAIL(GPT_ERR_INVALID_ARG, "n_tensors is NULL");
  const int n = 2 + 6 * D.L;
  *n_tensors = n;
  if (!offsets || capacity < n) FAIL(GPT_ERR_INVALID_ARG, "offsets NULL or capacity < 2 + 6*depth");
  const ParamLayout P = param_layout(D);
  int i = 0;
  offsets[i++] = P.wte;
  for (int l = 0; l < D.L; ++l) {
    const size_t b = P.qkv(D, l);
    for (int j = 0; j < 4; ++j) offsets[i++] = b + (size_t)j * D.d * D.d;
  }
  for (int l = 0; l < D.L; ++l) offsets[i++] = P.fc(D, l);
  for (int l = 0; l < D.L; ++l) offsets[i++] = P.proj(D, l);
  offsets[i++] = P.lm_head;
  return GPT_OK;
}

// ---------------------------------------------------------------------------
// component: GEMM
// ---------------------------------------------------------------------------
extern "C" gpt_status gpt_op_gemm(int32_t M, int32_t N, int32_t K, int32_t batch, const uint16_t* A,
                                  int32_t a_layout, int64_t lda, int64_t stride_a, const uint16_t* B,
                                  int32_t b_layout, int64_t ldb, int64_t stride_b, void* C,
                                  int32_t c_dtype, int64_t ldc, int64_t stride_c, float alpha,
                                  float beta, gpt_stream_t stream) {
  if (M < 0 || N < 0 || K < 0 || batch < 0) FAIL(GPT_ERR_INVALID_ARG, "negative size");
  if (M == 0 || N == 0 || batch == 0) return GPT_OK;
  if (!A || !B || !C) FAIL(GPT_ERR_INVALID_ARG, "NULL operand");
  if ((a_layout != GPT_LAYOUT_K_CONTIG && a_layout != GPT_LAYOUT_MN_CONTIG) ||
      (b_layout != GPT_LAYOUT_K_CONTIG && b_layout != GPT_LAYOUT_MN_CONTIG))
    FAIL(GPT_ERR_UNSUPPORTED, "unknown operand layout");
  if (c_dtype != GPT_DTYPE_F32 && c_dtype != GPT_DTYPE_BF16) FAIL(GPT_ERR_UNSUPPORTED, "unknown C dtype");
  if (c_dtype == GPT_DTYPE_BF16 && beta != 0.f) FAIL(GPT_ERR_INVALID_ARG, "beta must be 0 for bf16 C");
  if ((lda % 8) || (ldb % 8) || (ldc % 4) || lda <= 0 || ldb <= 0 || ldc <= 0)
    FAIL(GPT_ERR_INVALID_ARG, "lda, ldb must be positive multiples of 8 and ldc of 4");
  if ((stride_a % 8) || (stride_b % 8) || (stride_c % 4)) FAIL(GPT_ERR_INVALID_ARG, "batch strides misaligned");
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 15) FAIL(GPT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const long long arows = a_layout == GPT_LAYOUT_K_CONTIG ? K : M;
  const long long brows = b_layout == GPT_LAYOUT_K_CONTIG ? K : N;
  if ((a_layout == GPT_LAYOUT_K_CONTIG ? lda < K : lda < M) || (b_layout == GPT_LAYOUT_K_CONTIG ? ldb < K : ldb < N) ||
      ldc < N)
    FAIL(GPT_ERR_INVALID_ARG, "leading dimension smaller than the row length");
  (void)arows;
  (void)brows;
  GemmArgs a;
  a.M = M; a.N = N; a.K = K; a.batch = batch;
  a.A = A; a.lda = lda; a.sA = stride_a; a.a_kcontig = a_layout == GPT_LAYOUT_K_CONTIG;
  a.B = B; a.ldb = ldb; a.sB = stride_b; a.b_kcontig = b_layout == GPT_LAYOUT_K_CONTIG;
  a.C = C; a.ldc = ldc; a.sC = stride_c;
  a.alpha = alpha; a.beta = beta;
  TRY(gemm_bf16(a, c_dtype == GPT_DTYPE_F32 ? EPI_F32 : EPI_BF16, S(stream)));
  return GPT_OK;
}


