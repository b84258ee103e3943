// C ABI of libgptstep: argument validation, parameter/workspace layout and
// the launch sequence of the training step.  Kernels live in the .hip files.

#include <math.h>
#include <algorithm>
#include <string.h>

#include <mutex>
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

extern "C" int32_t gpt_abi_version(void) { return 3; }

// ---------------------------------------------------------------------------
// shapes and layouts
// ---------------------------------------------------------------------------
namespace {

struct Dims {
  int L, d, H, hidden, V, T, B, prec;
  int Hkv, dkv, dqkv;  // key/value heads, their width 128 Hkv, and the [q | k | v] width d + 2 dkv
  int window, pat_len;
  uint32_t pat_long;
  uint32_t feat;  // GPT_FEAT_* bits
  long long N;  // tokens per step
  bool has(uint32_t bit) const { return (feat & bit) != 0; }
  bool ve_layer(int l) const { return has(GPT_FEAT_VALUE_EMBED) && (l % 2) == 0; }
  // left attention window of layer l (-1: full causal)
  int layer_window(int l) const {
    if (window <= 0 || pat_len <= 0) return -1;
    return ((pat_long >> (l % pat_len)) & 1u) ? -1 : window;
  }
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
  if (s->n_kv_head < 0 || (s->n_kv_head > 0 && o->H % s->n_kv_head))
    FAIL(GPT_ERR_SHAPE, "n_kv_head must divide n_head = 32*depth/64");
  if (s->window < 0) FAIL(GPT_ERR_SHAPE, "window must be >= 0");
  if (s->pattern_len < 0 || s->pattern_len > 32) FAIL(GPT_ERR_SHAPE, "pattern_len must be in [0, 32]");
  o->Hkv = s->n_kv_head > 0 ? s->n_kv_head : o->H;
  o->dkv = 128 * o->Hkv;
  o->dqkv = o->d + 2 * o->dkv;
  o->window = s->window;
  o->pat_len = s->pattern_len;
  o->pat_long = s->pattern_long;
  if (s->features & ~15u) FAIL(GPT_ERR_SHAPE, "unknown feature bits");
  o->feat = s->features;
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
  size_t qkv(const Dims& D, int l) const { return wte_end + (size_t)l * (2 * (size_t)D.d + 2 * (size_t)D.dkv) * D.d; }
  size_t wk(const Dims& D, int l) const { return qkv(D, l) + (size_t)D.d * D.d; }
  size_t wv(const Dims& D, int l) const { return wk(D, l) + (size_t)D.dkv * D.d; }
  size_t wo(const Dims& D, int l) const { return qkv(D, l) + (size_t)D.dqkv * D.d; }
  size_t fc(const Dims& D, int l) const { return s_end + (size_t)l * D.hidden * D.d; }
  size_t proj(const Dims& D, int l) const { return f_end + (size_t)l * D.d * D.hidden; }
  // record-model tensors (present when any feature bit is set); l even
  size_t ve(const Dims& D, int l) const { return lm_end + (size_t)(l / 2) * D.V * D.dkv; }
  size_t vg(const Dims& D, int l) const { return vg0 + (size_t)(l / 2) * D.Hkv * 32; }
  size_t resid_l(int l) const { return sc + l; }
  size_t x0lam(const Dims& D, int l) const { return sc + D.L + l; }
  size_t smear_w(const Dims& D) const { return sc + 2 * (size_t)D.L; }
  size_t smear_lam(const Dims& D) const { return sc + 2 * (size_t)D.L + 24; }
  size_t backout(const Dims& D) const { return sc + 2 * (size_t)D.L + 25; }
  size_t wte_end, s_end, f_end, p_end, lm_end, vg0, sc;
};

ParamLayout param_layout(const Dims& D) {
  ParamLayout p;
  p.wte = 0;
  p.wte_end = (size_t)D.V * D.d;
  p.s_end = p.wte_end + (size_t)D.L * (2 * (size_t)D.d + 2 * (size_t)D.dkv) * D.d;
  p.f_end = p.s_end + (size_t)D.L * D.hidden * D.d;
  p.p_end = p.f_end + (size_t)D.L * D.d * D.hidden;
  p.lm_head = p.p_end;
  p.lm_end = p.lm_head + (size_t)D.V * D.d;
  p.total = p.lm_end;
  p.vg0 = p.sc = p.lm_end;
  if (D.feat) {
    const size_t nve = (size_t)(D.L / 2);
    p.vg0 = p.lm_end + nve * D.V * D.dkv;
    p.sc = p.vg0 + nve * D.Hkv * 32;
    p.total = p.sc + 2 * (size_t)D.L + 32;  // resid, x0lam, w[24], lam, backout, 6 unused
  }
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
  const int n = 2 + 6 * D.L + (D.feat ? D.L + 6 : 0);
  *n_tensors = n;
  if (!offsets || capacity < n) FAIL(GPT_ERR_INVALID_ARG, "offsets NULL or capacity below the tensor count");
  const ParamLayout P = param_layout(D);
  int i = 0;
  offsets[i++] = P.wte;
  for (int l = 0; l < D.L; ++l) {
    offsets[i++] = P.qkv(D, l);
    offsets[i++] = P.wk(D, l);
    offsets[i++] = P.wv(D, l);
    offsets[i++] = P.wo(D, l);
  }
  for (int l = 0; l < D.L; ++l) offsets[i++] = P.fc(D, l);
  for (int l = 0; l < D.L; ++l) offsets[i++] = P.proj(D, l);
  offsets[i++] = P.lm_head;
  if (D.feat) {
    for (int l = 0; l < D.L; l += 2) offsets[i++] = P.ve(D, l);
    for (int l = 0; l < D.L; l += 2) offsets[i++] = P.vg(D, l);
    offsets[i++] = P.resid_l(0);
    offsets[i++] = P.x0lam(D, 0);
    offsets[i++] = P.smear_w(D);
    offsets[i++] = P.smear_lam(D);
    offsets[i++] = P.backout(D);
    offsets[i++] = P.backout(D) + 1;
  }
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



// ---------------------------------------------------------------------------
// component: fp8 quantisation and fp8 GEMM
// ---------------------------------------------------------------------------
extern "C" int32_t gpt_fp8_partials(int32_t rows, int32_t cols) {
  if (rows < 1 || cols < 1) return 1;
  return fp8_partials(rows, cols);
}

extern "C" gpt_status gpt_op_quantize_fp8(const void* x, int32_t x_dtype, int64_t ldx, int32_t rows, int32_t cols,
                                          int32_t fmt, float* scale, uint8_t* q, int64_t ldq, uint8_t* qt,
                                          int64_t ldqt, float* partial, gpt_stream_t stream) {
  if (rows < 0 || cols < 0) FAIL(GPT_ERR_INVALID_ARG, "negative size");
  if (rows == 0 || cols == 0) return GPT_OK;
  if (!x || !scale || !partial) FAIL(GPT_ERR_INVALID_ARG, "NULL pointer");
  if (x_dtype != GPT_DTYPE_F32 && x_dtype != GPT_DTYPE_BF16) FAIL(GPT_ERR_UNSUPPORTED, "unknown x dtype");
  if (fmt != GPT_FP8_E4M3 && fmt != GPT_FP8_E5M2) FAIL(GPT_ERR_UNSUPPORTED, "unknown fp8 format");
  if ((rows % 16) || (cols % 16)) FAIL(GPT_ERR_INVALID_ARG, "rows and cols must be multiples of 16");
  if ((long long)rows * cols / 4 >= (1LL << 31)) FAIL(GPT_ERR_INVALID_ARG, "tensor too large");
  if (ldx < cols || (ldx % 8)) FAIL(GPT_ERR_INVALID_ARG, "ldx must be >= cols and a multiple of 8");
  if (q && (ldq < cols || (ldq % 8))) FAIL(GPT_ERR_INVALID_ARG, "ldq must be >= cols and a multiple of 8");
  if (qt && (ldqt < rows || (ldqt % 16))) FAIL(GPT_ERR_INVALID_ARG, "ldqt must be >= rows and a multiple of 16");
  if (((uintptr_t)x & 15) || ((uintptr_t)q & 7) || ((uintptr_t)qt & 15))
    FAIL(GPT_ERR_INVALID_ARG, "misaligned pointer");
  TRY(quantize_fp8(x, x_dtype == GPT_DTYPE_F32, ldx, rows, cols, fmt, partial, scale, q, ldq, qt, ldqt, S(stream)));
  return GPT_OK;
}

extern "C" gpt_status gpt_op_gemm_fp8(int32_t M, int32_t N, int32_t K, const uint8_t* A, int32_t fmt_a,
                                      int32_t a_layout, int64_t lda, const uint8_t* B, int32_t fmt_b,
                                      int32_t b_layout, int64_t ldb, float* C, int64_t ldc, const float* scale_a,
                                      const float* scale_b, float beta, gpt_stream_t stream) {
  if (M < 0 || N < 0 || K < 0) FAIL(GPT_ERR_INVALID_ARG, "negative size");
  if (M == 0 || N == 0) return GPT_OK;
  if (!A || !B || !C || !scale_a || !scale_b) FAIL(GPT_ERR_INVALID_ARG, "NULL pointer");
  if ((fmt_a != GPT_FP8_E4M3 && fmt_a != GPT_FP8_E5M2) || (fmt_b != GPT_FP8_E4M3 && fmt_b != GPT_FP8_E5M2))
    FAIL(GPT_ERR_UNSUPPORTED, "unknown fp8 format");
  if ((a_layout != GPT_LAYOUT_K_CONTIG && a_layout != GPT_LAYOUT_MN_CONTIG) ||
      (b_layout != GPT_LAYOUT_K_CONTIG && b_layout != GPT_LAYOUT_MN_CONTIG))
    FAIL(GPT_ERR_INVALID_ARG, "unknown operand layout");
  const bool ak = a_layout == GPT_LAYOUT_K_CONTIG, bk = b_layout == GPT_LAYOUT_K_CONTIG;
  if (!(ak && bk) && !(fmt_a == GPT_FP8_E5M2 && fmt_b == GPT_FP8_E4M3 && !bk))
    FAIL(GPT_ERR_UNSUPPORTED, "m/n-contiguous fp8 operands: E5M2 x E4M3 with B m/n-contiguous only");
  if (K % 16) FAIL(GPT_ERR_INVALID_ARG, "K must be a multiple of 16");
  if ((!ak && M % 16) || (!bk && N % 16))
    FAIL(GPT_ERR_INVALID_ARG, "an m/n-contiguous operand needs its rows (M or N) a multiple of 16");
  if (lda < (ak ? K : M) || ldb < (bk ? K : N) || ldc < N || (lda % 16) || (ldb % 16) || (ldc % 4))
    FAIL(GPT_ERR_INVALID_ARG, "lda, ldb must cover the contiguous dimension and be multiples of 16; ldc >= N and a multiple of 4");
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 15) FAIL(GPT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  GemmArgs a;
  a.M = M; a.N = N; a.K = K;
  a.A = A; a.lda = lda; a.a_kcontig = ak; a.B = B; a.ldb = ldb; a.b_kcontig = bk;
  a.C = C; a.ldc = ldc; a.beta = beta;
  a.scale_a = scale_a; a.scale_b = scale_b;
  TRY(gemm_fp8(a, EPI_F32, fmt_a, fmt_b, S(stream)));
  return GPT_OK;
}

// ---------------------------------------------------------------------------
// per-category kernel timing with HIP events (off unless enabled)
// ---------------------------------------------------------------------------
namespace {

enum ProfCat {
  P_EMBED_FWD, P_RMSNORM_FWD, P_GEMM_QKV, P_ATTN_FWD, P_GEMM_O, P_GEMM_FC, P_GEMM_PROJ, P_CE_FWD,
  P_CE_REDUCE, P_CE_DZ, P_CE_DH, P_CE_DW, P_RMSNORM_BWD, P_PROJ_DGRAD, P_PROJ_WGRAD, P_FC_DGRAD,
  P_FC_WGRAD, P_O_DGRAD, P_O_WGRAD, P_ATTN_BWD_KV, P_ATTN_BWD_Q, P_QKV_DGRAD, P_QKV_WGRAD, P_EMBED_BWD,
  P_FILL, P_MUON_ELEMWISE, P_NS_GRAM, P_NS_POLY, P_NS_UPDATE, P_FP8_QUANT, P_ADAMW, P_FEATURES, P_COUNT
};
const char* kProfNames[P_COUNT] = {
    "embed_fwd", "rmsnorm_fwd", "gemm_qkv_rope_fwd", "attn_fwd", "gemm_o_fwd", "gemm_fc_relu2_fwd",
    "gemm_proj_fwd", "gemm_ce_fwd", "ce_reduce", "gemm_ce_dlogits", "gemm_ce_dh", "gemm_ce_dw",
    "rmsnorm_bwd", "gemm_proj_dgrad", "gemm_proj_wgrad", "gemm_fc_dgrad", "gemm_fc_wgrad",
    "gemm_o_dgrad", "gemm_o_wgrad", "attn_bwd_dkdv", "attn_bwd_dq", "gemm_qkv_dgrad", "gemm_qkv_wgrad",
    "embed_bwd", "fill", "muon_elementwise", "ns_gram", "ns_poly", "ns_update", "fp8_quant", "adamw", "features"};

struct Profiler {
  uint64_t mask = 0;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<std::pair<size_t, size_t>> marks[P_COUNT];
  hipEvent_t get() {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};
Profiler g_prof;

struct ProfScope {
  int cat;
  hipStream_t s;
  size_t b = 0;
  bool on;
  ProfScope(int c, hipStream_t st) : cat(c), s(st), on((g_prof.mask >> c) & 1) {
    if (on) {
      b = g_prof.used;
      hipEvent_t e = g_prof.get();
      if (!e) { on = false; return; }
      hipEventRecord(e, s);
    }
  }
  ~ProfScope() {
    if (on) {
      const size_t en = g_prof.used;
      hipEvent_t e = g_prof.get();
      if (!e) return;
      hipEventRecord(e, s);
      g_prof.marks[cat].push_back({b, en});
    }
  }
};

}  // namespace

extern "C" int32_t gpt_profile_num_categories(void) { return P_COUNT; }

extern "C" const char* gpt_profile_category_name(int32_t cat) {
  return (cat >= 0 && cat < P_COUNT) ? kProfNames[cat] : "";
}

extern "C" gpt_status gpt_profile_enable(uint64_t mask) {
  g_prof.mask = mask;
  return GPT_OK;
}

extern "C" gpt_status gpt_profile_reset(void) {
  for (auto& m : g_prof.marks) m.clear();
  g_prof.used = 0;
  return GPT_OK;
}

extern "C" gpt_status gpt_profile_read(int32_t cat, double* total_ms, int32_t* launches) {
  if (cat < 0 || cat >= P_COUNT || !total_ms || !launches) FAIL(GPT_ERR_INVALID_ARG, "bad profile query");
  double t = 0.0;
  for (const auto& pr : g_prof.marks[cat]) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(g_prof.pool[pr.second]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_prof.pool[pr.first], g_prof.pool[pr.second]);
    if (e != hipSuccess) FAIL(GPT_ERR_HIP, std::string("profile events: ") + hipGetErrorString(e));
    t += ms;
  }
  *total_ms = t;
  *launches = (int32_t)g_prof.marks[cat].size();
  return GPT_OK;
}


// ---------------------------------------------------------------------------
// workspace layout of the step
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kAlign = 256;
inline size_t al(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// The head works on vocabulary chunks of vocab_chunk columns.  The forward
// keeps exp(z - m) of every logit (fp16) chunk-major, [chunk][N][chunk_ld]; the
// backward turns one chunk at a time into dlogits [N][chunk_ld] (bf16).
inline int vocab_chunk(const Dims& D) { return D.V < 8192 ? D.V : 8192; }
inline int chunk_ld(const Dims& D) { return (vocab_chunk(D) + 7) / 8 * 8; }
inline int n_chunks(const Dims& D) { return (D.V + vocab_chunk(D) - 1) / vocab_chunk(D); }

// Tile width of every head-forward launch, fixed from the whole vocabulary so
// that all chunks agree on the (max, sum) column groups: one group per wave,
// half a tile.  8192 is a multiple of both widths, so chunks start on tiles.
inline int ce_tile(const Dims& D) {
  GemmArgs a;
  a.M = (int)D.N; a.N = D.V; a.K = D.d; a.batch = 1; a.k_split = 1;
  return gemm_tile_n(a);
}
inline int ce_group(const Dims& D) { return ce_tile(D) / 2; }
inline int ce_nparts(const Dims& D) { return ((D.V + ce_tile(D) - 1) / ce_tile(D)) * 2; }

inline size_t wgrad_part_elems(int M, int N, int K);

struct Layer {
  size_t h1, r1, qkv, rq, rk, att, lse, h2, r2, act;
  // fp8 precision only: E4M3 codes of the block-product inputs [N, cols]
  // (the forward product's A operand, kept for the weight gradient, which
  // reads them as stored) and of the weights [out, in] (forward B operand;
  // the data gradient reads them as stored)
  size_t h1q, attq, h2q, actq;
  size_t wqkv8, wo8, wfc8, wproj8;
  // record-model features: bf16 stream before the residual scaling; value-embedding gates [N, Hkv]
  size_t xin, vgate;
};

// per-layer fp8 scales (fmax / amax of the tensor)
enum Fp8Scale { SC_H1, SC_ATT, SC_H2, SC_ACT, SC_WQKV, SC_WO, SC_WFC, SC_WPROJ, SC_G_MLP, SC_DU, SC_G_ATT,
                SC_DQKV, SC_COUNT = 16 };

struct WS {
  size_t cs, x, hf, rf, part, zt, lse, row_loss, ez;
  std::vector<Layer> layer;
  // backward scratch
  size_t g, g_bf, dh, du, dout, delta, dqkv, dz, wpart, emb;
  // fp8 precision only: codes of the current output gradient [N, cols]
  // (backward); scales; amax partials
  size_t dyq, scales, qpart;
  // record-model features: smear sigmoids [N]; x0 and x_mid [N, d] fp32;
  // backward: gradient reaching x0 (g0), the head's stream gradient (gfin),
  // value-embedding gate gradients [N, Hkv], partial sums of the reductions
  size_t sig, x0, xmid, g0, gfin, dzve, fpart;
  size_t total;
};

WS ws_layout(const Dims& D) {
  WS w;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = al(o + bytes); return r; };
  const size_t N = (size_t)D.N, d = D.d, H = D.H, Hkv = D.Hkv, dq3 = D.dqkv;
  w.cs = take(2 * (size_t)D.T * 64 * 4);
  w.x = take(N * d * 4);
  w.layer.resize(D.L);
  for (int l = 0; l < D.L; ++l) {
    Layer& L = w.layer[l];
    L.h1 = take(N * d * 2);
    L.r1 = take(N * 4);
    L.qkv = take(N * dq3 * 2);
    L.rq = take(N * H * 4);
    L.rk = take(N * Hkv * 4);
    L.att = take(N * d * 2);
    L.lse = take(N * H * 4);
    L.h2 = take(N * d * 2);
    L.r2 = take(N * 4);
    L.act = take(N * D.hidden * 2);
  }
  w.hf = take(N * d * 2);
  w.rf = take(N * 4);
  w.part = take(N * (size_t)ce_nparts(D) * 8);
  w.ez = take((size_t)n_chunks(D) * N * (size_t)chunk_ld(D) * 2);
  w.zt = take(N * 4);
  w.lse = take(N * 4);
  w.row_loss = take(N * 4);
  w.g = take(N * d * 4);
  w.g_bf = take(N * d * 2);
  w.dh = take(N * d * 4);
  w.du = take(N * D.hidden * 2);
  w.dout = take(N * d * 2);
  w.delta = take(N * H * 4);
  w.emb = take(embed_bwd_workspace((long long)N, D.V));
  w.dqkv = take(N * dq3 * 2);
  w.dz = take(N * (size_t)chunk_ld(D) * 2);
  {
    const int Nt = (int)D.N, dd = D.d, hd = D.hidden;
    size_t mx = 0;
    mx = std::max(mx, wgrad_part_elems(D.dqkv, dd, Nt));
    mx = std::max(mx, wgrad_part_elems(dd, dd, Nt));
    mx = std::max(mx, wgrad_part_elems(hd, dd, Nt));
    mx = std::max(mx, wgrad_part_elems(dd, hd, Nt));
    mx = std::max(mx, wgrad_part_elems(vocab_chunk(D), dd, Nt));
    w.wpart = take(std::max<size_t>(mx, 1) * 4);
  }
  w.sig = w.x0 = w.xmid = w.g0 = w.gfin = w.dzve = w.fpart = 0;
  for (int l = 0; l < D.L; ++l) w.layer[l].xin = w.layer[l].vgate = 0;
  if (D.feat) {
    const size_t Nd = N * d;
    w.sig = take(N * 4);
    w.fpart = take((size_t)feature_partial_floats(D.Hkv) * 4);
    if (D.has(GPT_FEAT_RESID_LAMBDA)) {
      w.x0 = take(Nd * 4);
      w.g0 = take(Nd * 4);
      for (int l = 0; l < D.L; ++l) w.layer[l].xin = take(Nd * 2);
    }
    if (D.has(GPT_FEAT_BACKOUT)) {
      w.xmid = take(Nd * 4);
      w.gfin = take(Nd * 4);
    }
    if (D.has(GPT_FEAT_VALUE_EMBED)) {
      w.dzve = take(N * Hkv * 4);
      for (int l = 0; l < D.L; l += 2) w.layer[l].vgate = take(N * Hkv * 4);
    }
  }
  w.dyq = w.scales = w.qpart = 0;
  if (D.prec == GPT_PREC_FP8) {
    const size_t dd = (size_t)d * d, hd = (size_t)D.hidden;
    for (int l = 0; l < D.L; ++l) {
      Layer& L = w.layer[l];
      L.h1q = take(N * d);
      L.attq = take(N * d);
      L.h2q = take(N * d);
      L.actq = take(N * hd);
      L.wqkv8 = take((size_t)D.dqkv * d);
      L.wo8 = take(dd);
      L.wfc8 = take(hd * d);
      L.wproj8 = take(hd * d);
    }
    w.dyq = take(N * hd);
    w.scales = take((size_t)D.L * SC_COUNT * 4);
    // amax partials: the standalone reduction, one per row (norm kernels), or
    // one per wave of the [N, 4d] bf16 products
    GemmArgs ga;
    ga.M = (int)D.N; ga.N = D.hidden; ga.K = d;
    long long slots = std::max<long long>(std::max<long long>(kFp8Partials, (long long)D.N), gemm_amax_slots(ga));
    slots = std::max(slots, std::max(attn_fwd_amax_slots(D.B, D.H, D.T), attn_bwd_amax_slots(D.B, D.H, D.Hkv, D.T)));
    slots = std::max(slots, (long long)D.L * kFp8Partials);  // the batched weight quantisation
    w.qpart = take((size_t)slots * 4);
  }
  w.total = o;
  return w;
}

template <class T>
inline T* at(void* ws, size_t off) { return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off); }

// k-splits for a weight-gradient product (small output, long K): each split
// writes a partial that a small reduction adds up (no atomics,
// deterministic), at least 2048 k per split.  Outputs of at least 256 x 256
// take 256 x 256 tiles (one workgroup per CU) and the split count that
// minimises the modelled time rounds(ks) / ks + 0.008 ks: the waves of
// workgroups the launch needs over the work each workgroup does, plus the
// partial traffic and per-workgroup overhead that grow with the count (fit to
// the d20 products, measured without the reduction: the output projection's
// 25 tiles take 10 splits, 0.196 ms against 0.264 ms with 128 x 128 tiles; the
// q/k/v product's 75 take 3, 0.557 against 0.617 ms with 10; the MLP
// products' 100 take 5).  Smaller outputs take 128 x 128 tiles (two
// workgroups per CU) and the smallest count whose last wave is within 2.5 %
// of the best fill.
struct WgradPlan {
  int ks;    // k splits (1: none)
  int tile;  // forced tile width (0: the launch's own choice)
};
inline WgradPlan wgrad_plan(int M, int N, int K) {
  const int kmax = std::max(1, std::min(32, K / 2048));
  if (M >= 256 && N >= 256) {
    const long long t256 = (long long)((M + 255) / 256) * ((N + 255) / 256);
    if (t256 >= 256) return {1, 0};
    double best = 1e30;
    int bk = 1;
    for (int ks = 1; ks <= kmax; ++ks) {
      const double rounds = (double)((t256 * ks + 255) / 256);
      const double cost = rounds / ks + 0.008 * ks;
      if (cost < best - 1e-9) { best = cost; bk = ks; }
    }
    return {bk, 256};
  }
  const long long t128 = (long long)((M + 127) / 128) * ((N + 127) / 128);
  const int hi = std::min(16, kmax);
  auto fill = [&](int ks) {
    const long long b = t128 * ks;
    return (double)b / (double)(((b + 511) / 512) * 512);
  };
  double best = 0.0;
  for (int ks = 1; ks <= hi; ++ks) best = std::max(best, fill(ks));
  for (int ks = 1; ks <= hi; ++ks)
    if (fill(ks) >= best - 0.025) return {ks, 128};
  return {1, 128};
}

inline size_t wgrad_part_elems(int M, int N, int K) {
  const int ks = wgrad_plan(M, N, K).ks;
  return ks > 1 ? (size_t)ks * M * N : 0;
}

// C[M,N] (f32, dense, ld N) (+)= A^T B with A stored [K][M], B stored [K][N] (bf16)
int wgrad(const void* A, long long lda, const void* B, long long ldb, float* C, int M, int N, int K,
          bool accumulate, float* part, hipStream_t s) {
  GemmArgs a;
  a.M = M; a.N = N; a.K = K;
  a.A = A; a.lda = lda; a.a_kcontig = 0;
  a.B = B; a.ldb = ldb; a.b_kcontig = 0;
  const WgradPlan pl = wgrad_plan(M, N, K);
  a.tile = pl.tile;
  if (pl.ks == 1) {
    a.C = C; a.ldc = N;
    a.beta = accumulate ? 1.f : 0.f;
    return gemm_bf16(a, EPI_F32, s);
  }
  a.C = part; a.ldc = N; a.k_split = pl.ks; a.split_stride = (long long)M * N; a.beta = 0.f;
  int rc = gemm_bf16(a, EPI_F32, s);
  if (rc) return rc;
  return launch_splitk_reduce(part, pl.ks, (long long)M * N, C, nullptr, (long long)M * N, accumulate ? 1.f : 0.f, s);
}

// fp8 weight gradient: C[M,N] (+)= dY^T X / (sa sb) from the codes as
// stored: dY [K][M] (E5M2) and X [K][N] (E4M3), both m/n-contiguous
int wgrad_fp8(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb, float* C, int M, int N, int K,
              bool accumulate, float* part, hipStream_t s) {
  GemmArgs a;
  a.M = M; a.N = N; a.K = K;
  a.A = A; a.lda = M; a.a_kcontig = 0; a.B = B; a.ldb = N; a.b_kcontig = 0;
  a.scale_a = sa; a.scale_b = sb;
  const WgradPlan pl = wgrad_plan(M, N, K);
  a.tile = pl.tile;
  if (pl.ks == 1) {
    a.C = C; a.ldc = N;
    a.beta = accumulate ? 1.f : 0.f;
    return gemm_fp8(a, EPI_F32, 1, 0, s);
  }
  a.C = part; a.ldc = N; a.k_split = pl.ks; a.split_stride = (long long)M * N; a.beta = 0.f;
  int rc = gemm_fp8(a, EPI_F32, 1, 0, s);
  if (rc) return rc;
  return launch_splitk_reduce(part, pl.ks, (long long)M * N, C, nullptr, (long long)M * N, accumulate ? 1.f : 0.f, s);
}

}  // namespace

extern "C" gpt_status gpt_workspace_size(const gpt_shape* shape, size_t* bytes) {
  Dims D;
  TRY(check_shape(shape, &D));
  if (!bytes) FAIL(GPT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ws_layout(D).total;
  return GPT_OK;
}

extern "C" gpt_status gpt_workspace_tensor(const gpt_shape* shape, int32_t which, int32_t layer, size_t* offset,
                                           size_t* bytes) {
  Dims D;
  TRY(check_shape(shape, &D));
  if (!offset || !bytes) FAIL(GPT_ERR_INVALID_ARG, "NULL output");
  const WS w = ws_layout(D);
  const size_t N = (size_t)D.N, d = D.d;
  if (which >= 1 && which <= 5 && (layer < 0 || layer >= D.L)) FAIL(GPT_ERR_INVALID_ARG, "layer out of range");
  switch (which) {
    case 0: *offset = w.x; *bytes = N * d * 4; break;
    case 1: *offset = w.layer[layer].h1; *bytes = N * d * 2; break;
    case 2: *offset = w.layer[layer].qkv; *bytes = N * (size_t)D.dqkv * 2; break;
    case 3: *offset = w.layer[layer].att; *bytes = N * d * 2; break;
    case 4: *offset = w.layer[layer].h2; *bytes = N * d * 2; break;
    case 5: *offset = w.layer[layer].act; *bytes = N * D.hidden * 2; break;
    case 6: *offset = w.hf; *bytes = N * d * 2; break;
    case 7: *offset = w.lse; *bytes = N * 4; break;
    case 8: *offset = w.row_loss; *bytes = N * 4; break;
    case 9: *offset = w.zt; *bytes = N * 4; break;
    default: FAIL(GPT_ERR_INVALID_ARG, "unknown workspace tensor");
  }
  return GPT_OK;
}

extern "C" gpt_status gpt_cast_bf16(const float* src, uint16_t* dst, size_t n, gpt_stream_t stream) {
  if (n == 0) return GPT_OK;
  if (!src || !dst) FAIL(GPT_ERR_INVALID_ARG, "NULL pointer");
  if (((uintptr_t)src & 15) || ((uintptr_t)dst & 7)) FAIL(GPT_ERR_INVALID_ARG, "src must be 16-byte and dst 8-byte aligned");
  TRY(launch_cast_bf16(src, dst, (long long)n, S(stream)));
  return GPT_OK;
}

namespace {

int check_step_args(const gpt_shape* shape, const gpt_params* params, const int32_t* ids, void* ws,
                    size_t ws_bytes, Dims* D, WS* w) {
  int rc = check_shape(shape, D);
  if (rc) return rc;
  if (!params || !params->bf16) FAIL(GPT_ERR_INVALID_ARG, "params or params->bf16 is NULL");
  if (!ids) FAIL(GPT_ERR_INVALID_ARG, "ids is NULL");
  if (!ws) FAIL(GPT_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)ws % kAlign) FAIL(GPT_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (((uintptr_t)params->bf16 & 15)) FAIL(GPT_ERR_INVALID_ARG, "params->bf16 must be 16-byte aligned");
  *w = ws_layout(*D);
  if (ws_bytes < w->total) FAIL(GPT_ERR_WORKSPACE, "workspace smaller than gpt_workspace_size()");
  if (D->prec == GPT_PREC_FP8 && (D->N % 16))
    FAIL(GPT_ERR_UNSUPPORTED, "fp8 precision needs batch*seq_len to be a multiple of 16");
  return 0;
}

}  // namespace

extern "C" gpt_status gpt_step_fwd(const gpt_shape* shape, const gpt_params* params, const int32_t* ids,
                                   float* loss, float* row_lse, float* logits, void* ws, size_t ws_bytes,
                                   gpt_stream_t stream) {
  Dims D;
  WS w;
  TRY(check_step_args(shape, params, ids, ws, ws_bytes, &D, &w));
  if (!loss) FAIL(GPT_ERR_INVALID_ARG, "loss is NULL");
  if (logits && (D.V % 4)) FAIL(GPT_ERR_INVALID_ARG, "logits output needs vocab % 4 == 0");
  hipStream_t s = S(stream);
  const ParamLayout P = param_layout(D);
  const uint16_t* W = params->bf16;
  const int N = (int)D.N, d = D.d;
  float* x = at<float>(ws, w.x);
  float* cs = at<float>(ws, w.cs);

  TRY(launch_rope_table(cs, D.T, s));
  const bool f8 = D.prec == GPT_PREC_FP8;
  const int hid = D.hidden;
  float* qpart = f8 ? at<float>(ws, w.qpart) : nullptr;
  const uint8_t* xq = nullptr;  // codes of the current product input
  if (f8) {
    // E4M3 codes of every block weight, one scale per tensor: one batched
    // launch per weight kind over all layers (same shape, a fixed stride apart
    // in the packed parameters and in the per-layer workspace)
    ProfScope ps_(P_FP8_QUANT, s);
    float* sc0 = at<float>(ws, w.scales);
    auto kind = [&](auto poff, size_t Layer::*q8, int rows, int cols, int sc_slot) -> int {
      const long long sx = (long long)(poff(1) - poff(0));
      const long long sq = (long long)(w.layer[1].*q8 - w.layer[0].*q8);
      bool uniform = true;
      for (int l = 1; l < D.L; ++l)
        uniform = uniform && (long long)(poff(l) - poff(0)) == l * sx &&
                  (long long)(w.layer[l].*q8 - w.layer[0].*q8) == l * sq;
      // one launch for all layers, or (were the strides not uniform) one per layer
      const int cnt = uniform ? D.L : 1;
      for (int l0 = 0; l0 < D.L; l0 += cnt) {
        const Layer& L = w.layer[l0];
        float* scl = sc0 + (size_t)l0 * SC_COUNT + sc_slot;
        TRY(launch_fp8_amax_scale(W + poff(l0), 0, cols, rows, cols, 0, qpart, scl, s, cnt, sx, SC_COUNT));
        TRY(launch_fp8_quant(W + poff(l0), 0, cols, rows, cols, 0, scl, at<uint8_t>(ws, L.*q8), cols, nullptr, 0,
                             s, cnt, sx, SC_COUNT, sq));
      }
      return 0;
    };
    TRY(kind([&](int l) { return P.qkv(D, l); }, &Layer::wqkv8, D.dqkv, d, SC_WQKV));
    TRY(kind([&](int l) { return P.wo(D, l); }, &Layer::wo8, d, d, SC_WO));
    TRY(kind([&](int l) { return P.fc(D, l); }, &Layer::wfc8, hid, d, SC_WFC));
    TRY(kind([&](int l) { return P.proj(D, l); }, &Layer::wproj8, d, hid, SC_WPROJ));
  }
  // y (op)= X W^T for one block product: bf16 operands, or (fp8) the E4M3 codes
  // of X (quantised here into the layer's buffer, which the weight gradient
  // reads again) and of W
  // np > 0: the producer already wrote np amax partials into qpart
  auto quant_x = [&](const uint16_t* X, int K, size_t xq_off, float* sx, long long np) -> int {
    if (!f8) return 0;
    ProfScope ps_(P_FP8_QUANT, s);
    uint8_t* q = at<uint8_t>(ws, xq_off);
    xq = q;
    if (np > 0) return quantize_fp8_partials(X, 0, K, N, K, 0, qpart, np, sx, q, K, nullptr, 0, s);
    return quantize_fp8(X, 0, K, N, K, 0, qpart, sx, q, K, nullptr, 0, s);
  };
  auto block_fwd = [&](GemmArgs& a, int epi, int K, const uint8_t* w8, const float* sx, const float* sw) -> int {
    if (!f8) return gemm_bf16(a, epi, s);
    a.A = xq; a.lda = K; a.B = w8; a.ldb = K;
    a.scale_a = sx; a.scale_b = sw;
    return gemm_fp8(a, epi, 0, 0, s);
  };
  const bool f_resid = D.has(GPT_FEAT_RESID_LAMBDA), f_smear = D.has(GPT_FEAT_SMEAR);
  const bool f_back = D.has(GPT_FEAT_BACKOUT);
  float* x0 = f_resid ? at<float>(ws, w.x0) : nullptr;
  float* xmid = f_back ? at<float>(ws, w.xmid) : nullptr;
  {
    ProfScope ps_(P_EMBED_FWD, s);
    if (f_smear || f_resid)  // gather (+ smear with the previous token), x0 kept for the residual scalars
      TRY(launch_smear_fwd(ids, W + P.wte, f_smear ? W + P.smear_w(D) : nullptr, f_smear ? W + P.smear_lam(D) : nullptr,
                           x, x0, at<float>(ws, w.sig), D.B, D.T, d, D.V, s));
    else
      TRY(launch_embed_fwd(ids, W + P.wte, x, D.B, D.T, d, D.V, s));
  }
  long long act_slots = 0;
  for (int l = 0; l < D.L; ++l) {
    const Layer& L = w.layer[l];
    float* sc = f8 ? at<float>(ws, w.scales) + (size_t)l * SC_COUNT : nullptr;
    uint16_t* h1 = at<uint16_t>(ws, L.h1);
    uint16_t* qkv = at<uint16_t>(ws, L.qkv);
    uint16_t* att = at<uint16_t>(ws, L.att);
    uint16_t* h2 = at<uint16_t>(ws, L.h2);
    uint16_t* act = at<uint16_t>(ws, L.act);
    {
      ProfScope ps_(P_RMSNORM_FWD, s);
      if (f_resid)  // x <- resid_l x + x0lam_l x0, then the norm
        TRY(launch_mix_rmsnorm_fwd(x, x0, W + P.resid_l(l), W + P.x0lam(D, l), 1.f, at<uint16_t>(ws, L.xin), h1,
                                   at<float>(ws, L.r1), N, d, qpart, s));
      else
        TRY(launch_rmsnorm_fwd(x, h1, at<float>(ws, L.r1), N, d, s, qpart));
    }
    TRY(quant_x(h1, d, L.h1q, sc ? sc + SC_H1 : nullptr, N));
    {
      GemmArgs a;  // [q | k | v] = h1 [Wq; Wk; Wv]^T, q and k rotated and RMS-normalised per head
      ProfScope ps_(P_GEMM_QKV, s);
      a.M = N; a.N = D.dqkv; a.K = d;
      a.A = h1; a.lda = d; a.B = W + P.qkv(D, l); a.ldb = d;
      a.C = qkv; a.ldc = D.dqkv;
      a.rope = cs; a.row_T = D.T; a.n_head = D.H; a.n_kv_head = D.Hkv;
      a.part = at<float>(ws, L.rq); a.zt = at<float>(ws, L.rk);
      TRY(block_fwd(a, EPI_QKV, d, f8 ? at<uint8_t>(ws, L.wqkv8) : nullptr, sc ? sc + SC_H1 : nullptr,
                    sc ? sc + SC_WQKV : nullptr));
    }
    if (D.ve_layer(l)) {  // v += 3 sigmoid(h1[:32] Wg^T) VE[token] per key/value head
      ProfScope ps_(P_FEATURES, s);
      TRY(launch_ve_fwd(ids, h1, d, W + P.vg(D, l), W + P.ve(D, l), qkv + d + D.dkv, D.dqkv, at<float>(ws, L.vgate),
                        D.B, D.T, D.Hkv, D.V, s));
    }
    {
      // fp8: the kernel also leaves the per-wave amax partials of its output
      ProfScope ps_(P_ATTN_FWD, s);
      TRY(launch_attn_fwd(qkv, qkv + d, qkv + d + D.dkv, D.dqkv, att, d, at<float>(ws, L.lse), D.B, D.H, D.Hkv, D.T,
                          D.layer_window(l), s, true, qpart));
    }
    TRY(quant_x(att, d, L.attq, sc ? sc + SC_ATT : nullptr, f8 ? attn_fwd_amax_slots(D.B, D.H, D.T) : 0));
    {
      GemmArgs a;  // x += att Wo^T
      ProfScope ps_(P_GEMM_O, s);
      a.M = N; a.N = d; a.K = d;
      a.A = att; a.lda = d; a.B = W + P.wo(D, l); a.ldb = d;
      a.C = x; a.ldc = d;
      TRY(block_fwd(a, EPI_RESID, d, f8 ? at<uint8_t>(ws, L.wo8) : nullptr, sc ? sc + SC_ATT : nullptr,
                    sc ? sc + SC_WO : nullptr));
    }
    { ProfScope ps_(P_RMSNORM_FWD, s); TRY(launch_rmsnorm_fwd(x, h2, at<float>(ws, L.r2), N, d, s, qpart)); }
    TRY(quant_x(h2, d, L.h2q, sc ? sc + SC_H2 : nullptr, N));
    {
      GemmArgs a;  // act = relu(h2 Wfc^T)^2
      ProfScope ps_(P_GEMM_FC, s);
      a.M = N; a.N = hid; a.K = d;
      a.A = h2; a.lda = d; a.B = W + P.fc(D, l); a.ldb = d;
      a.C = act; a.ldc = hid;
      a.amax = qpart;  // NULL for bf16
      act_slots = f8 ? gemm_amax_slots(a) : 0;
      TRY(block_fwd(a, EPI_RELU2, d, f8 ? at<uint8_t>(ws, L.wfc8) : nullptr, sc ? sc + SC_H2 : nullptr,
                    sc ? sc + SC_WFC : nullptr));
    }
    TRY(quant_x(act, hid, L.actq, sc ? sc + SC_ACT : nullptr, act_slots));
    {
      GemmArgs a;  // x += act Wproj^T
      ProfScope ps_(P_GEMM_PROJ, s);
      a.M = N; a.N = d; a.K = hid;
      a.A = act; a.lda = hid; a.B = W + P.proj(D, l); a.ldb = hid;
      a.C = x; a.ldc = d;
      TRY(block_fwd(a, EPI_RESID, hid, f8 ? at<uint8_t>(ws, L.wproj8) : nullptr,
                    sc ? sc + SC_ACT : nullptr, sc ? sc + SC_WPROJ : nullptr));
    }
    if (f_back && l == D.L / 2 - 1) {  // the middle stream, for backout
      ProfScope ps_(P_FEATURES, s);
      auto copy = [&]() -> int {
        GS_HIP_CHECK(hipMemcpyAsync(xmid, x, (size_t)N * d * 4, hipMemcpyDeviceToDevice, s));
        return 0;
      };
      TRY(copy());
    }
  }
  uint16_t* hf = at<uint16_t>(ws, w.hf);
  {
    ProfScope ps_(P_RMSNORM_FWD, s);
    if (f_back)  // x <- x - backout x_mid, then the final norm
      TRY(launch_mix_rmsnorm_fwd(x, xmid, nullptr, W + P.backout(D), -1.f, nullptr, hf, at<float>(ws, w.rf), N, d,
                                 nullptr, s));
    else
      TRY(launch_rmsnorm_fwd(x, hf, at<float>(ws, w.rf), N, d, s));
  }
  for (int c0 = 0; c0 < D.V; c0 += vocab_chunk(D)) {
    // per-wave (max m, sum exp) of the logits hf W_lm^T and the target logit;
    // exp(z - m) is kept (fp16) for the backward
    GemmArgs a;
    ProfScope ps_(P_CE_FWD, s);
    a.M = N; a.N = std::min(vocab_chunk(D), D.V - c0); a.K = d;
    a.A = hf; a.lda = d; a.B = W + P.lm_head + (size_t)c0 * d; a.ldb = d;
    a.C = at<uint16_t>(ws, w.ez) + (size_t)c0 * N; a.ldc = chunk_ld(D);  // chunk c0 / vocab_chunk
    a.row_i = ids; a.row_T = D.T; a.col_offset = c0;
    a.part = at<float>(ws, w.part) + (size_t)(c0 / ce_tile(D)) * 4; a.nparts = ce_nparts(D);
    a.zt = at<float>(ws, w.zt);
    a.tile = ce_tile(D);
    TRY(gemm_bf16(a, EPI_CE_FWD, s));
  }
  { ProfScope ps_(P_CE_REDUCE, s); TRY(launch_ce_reduce(at<float>(ws, w.part), ce_nparts(D), at<float>(ws, w.zt), at<float>(ws, w.lse),
                       at<float>(ws, w.row_loss), row_lse, N, s)); }
  { ProfScope ps_(P_CE_REDUCE, s); TRY(launch_loss_mean(at<float>(ws, w.row_loss), loss, N, s)); }
  if (logits) {
    GemmArgs a;
    a.M = N; a.N = D.V; a.K = d;
    a.A = hf; a.lda = d; a.B = W + P.lm_head; a.ldb = d;
    a.C = logits; a.ldc = D.V;
    TRY(gemm_bf16(a, EPI_F32, s));
  }
  return GPT_OK;
}

extern "C" gpt_status gpt_step_bwd(const gpt_shape* shape, const gpt_params* params, const int32_t* ids,
                                   int32_t accumulate, void* ws, size_t ws_bytes, gpt_stream_t stream) {
  if (!shape) FAIL(GPT_ERR_INVALID_ARG, "shape is NULL");
  const double n = (double)shape->batch * (double)shape->seq_len;
  return gpt_step_bwd_scaled(shape, params, ids, accumulate, n > 0 ? (float)(1.0 / n) : 1.f, ws, ws_bytes, stream);
}

extern "C" gpt_status gpt_step_bwd_scaled(const gpt_shape* shape, const gpt_params* params, const int32_t* ids,
                                          int32_t accumulate, float loss_scale, void* ws, size_t ws_bytes,
                                          gpt_stream_t stream) {
  Dims D;
  WS w;
  TRY(check_step_args(shape, params, ids, ws, ws_bytes, &D, &w));
  if (!(loss_scale > 0.f) || !isfinite(loss_scale)) FAIL(GPT_ERR_INVALID_ARG, "loss_scale must be positive and finite");
  if (!params->grad) FAIL(GPT_ERR_INVALID_ARG, "params->grad is NULL");
  if ((uintptr_t)params->grad & 15) FAIL(GPT_ERR_INVALID_ARG, "params->grad must be 16-byte aligned");
  if (accumulate != 0 && accumulate != 1) FAIL(GPT_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  hipStream_t s = S(stream);
  const ParamLayout P = param_layout(D);
  const uint16_t* W = params->bf16;
  float* G = params->grad;
  const bool acc = accumulate != 0;
  const int N = (int)D.N, d = D.d, hid = D.hidden;
  uint16_t* hf = at<uint16_t>(ws, w.hf);
  float* g = at<float>(ws, w.g);
  uint16_t* g_bf = at<uint16_t>(ws, w.g_bf);
  float* dh = at<float>(ws, w.dh);                    // the head's data gradient (fp32, summed over vocabulary chunks)
  uint16_t* dh16 = reinterpret_cast<uint16_t*>(dh);  // the blocks' (bf16 product outputs), same memory
  uint16_t* du = at<uint16_t>(ws, w.du);
  uint16_t* dout = at<uint16_t>(ws, w.dout);
  uint16_t* dqkv = at<uint16_t>(ws, w.dqkv);
  uint16_t* dz = at<uint16_t>(ws, w.dz);
  float* wpart = at<float>(ws, w.wpart);
  const float* cs = at<float>(ws, w.cs);
  const bool f_resid = D.has(GPT_FEAT_RESID_LAMBDA), f_smear = D.has(GPT_FEAT_SMEAR);
  const bool f_back = D.has(GPT_FEAT_BACKOUT);
  const long long Nd = (long long)N * d;
  float* fpart = D.feat ? at<float>(ws, w.fpart) : nullptr;
  float* g0 = f_resid ? at<float>(ws, w.g0) : nullptr;
  float* gfin = f_back ? at<float>(ws, w.gfin) : nullptr;
  float* dzve = D.has(GPT_FEAT_VALUE_EMBED) ? at<float>(ws, w.dzve) : nullptr;
  if (D.feat && !acc) {
    // the value-embedding tables are gathered onto these zeros; a cleared feature bit leaves its gradients at 0
    ProfScope ps_(P_FILL, s);
    TRY(launch_fill_f32(G + P.lm_end, (long long)(P.total - P.lm_end), 0.f, s));
  }
  if (D.has(GPT_FEAT_VALUE_EMBED)) {
    // the token ids' stable sort, shared by the value-embedding tables and the token embedding
    ProfScope ps_(P_EMBED_BWD, s);
    TRY(launch_embed_sort(ids, D.B, D.T, D.V, at<void>(ws, w.emb), s));
  }

  // head + cross-entropy backward from the exponentials the forward kept, one
  // vocabulary chunk at a time: dz = bf16(loss_scale (softmax(z) - onehot(target))),
  // dh (+)= dz W_lm[chunk], dW_lm[chunk] (+)= dz^T hf
  const int lz = chunk_ld(D);
  for (int c0 = 0; c0 < D.V; c0 += vocab_chunk(D)) {
    const int nv = std::min(vocab_chunk(D), D.V - c0);
    {
      ProfScope ps_(P_CE_DZ, s);
      TRY(launch_ce_dz(at<uint16_t>(ws, w.ez) + (size_t)c0 * N, dz, at<float>(ws, w.part), ce_nparts(D), ce_group(D),
                       c0, at<float>(ws, w.lse), ids, D.T, N, nv, lz, loss_scale, s));
    }
    {
      GemmArgs a;
      ProfScope ps_(P_CE_DH, s);
      a.M = N; a.N = d; a.K = nv;
      a.A = dz; a.lda = lz; a.B = W + P.lm_head + (size_t)c0 * d; a.ldb = d; a.b_kcontig = 0;
      a.C = dh; a.ldc = d; a.beta = c0 > 0 ? 1.f : 0.f;
      TRY(gemm_bf16(a, EPI_F32, s));
    }
    { ProfScope ps_(P_CE_DW, s); TRY(wgrad(dz, lz, hf, d, G + P.lm_head + (size_t)c0 * d, nv, d, N, acc, wpart, s)); }
  }
  { ProfScope ps_(P_FILL, s); TRY(launch_fill_f32(g, (long long)N * d, 0.f, s)); }
  const bool f8 = D.prec == GPT_PREC_FP8;
  float* qpart = f8 ? at<float>(ws, w.qpart) : nullptr;
  { ProfScope ps_(P_RMSNORM_BWD, s); TRY(launch_rmsnorm_bwd(dh, false, hf, at<float>(ws, w.rf), g, g_bf, N, d, s, qpart)); }
  if (f_back) {  // x_final = x_L - backout x_mid: d backout = -g . x_mid; g is kept for the middle layer
    ProfScope ps_(P_FEATURES, s);
    TRY(launch_backout_bwd(g, at<float>(ws, w.xmid), gfin, Nd, fpart, G + P.backout(D), acc, s));
  }
  // the per-row amax partials of g_bf (fp8) are valid only right after a norm backward wrote them
  bool g_amax_ok = true;

  uint8_t* dyq = f8 ? at<uint8_t>(ws, w.dyq) : nullptr;
  // E5M2 codes of an output gradient dY [N, cols] (the data gradient reads
  // them k-contiguous, the weight gradient m-contiguous)
  // np > 0: the producer already wrote np amax partials into qpart
  auto quant_dy = [&](const uint16_t* dy, int cols, float* sdy, long long np) -> int {
    ProfScope ps_(P_FP8_QUANT, s);
    if (np > 0) return quantize_fp8_partials(dy, 0, cols, N, cols, 1, qpart, np, sdy, dyq, cols, nullptr, 0, s);
    return quantize_fp8(dy, 0, cols, N, cols, 1, qpart, sdy, dyq, cols, nullptr, 0, s);
  };
  // data gradient dX [N, cols_x] = dY W for a weight W [cols_dy, cols_x]: fp8
  // operands are the dY codes and the weight codes as stored (n-contiguous)
  auto dgrad_fp8 = [&](GemmArgs& a, int epi, int cols_dy, int cols_x, const uint8_t* w8, const float* sdy,
                       const float* sw) -> int {
    a.A = dyq; a.lda = cols_dy; a.a_kcontig = 1;
    a.B = w8; a.ldb = cols_x; a.b_kcontig = 0;
    a.scale_a = sdy; a.scale_b = sw;
    return gemm_fp8(a, epi, 1, 0, s);
  };

  long long du_slots = 0;
  for (int l = D.L - 1; l >= 0; --l) {
    const Layer& L = w.layer[l];
    float* sc = f8 ? at<float>(ws, w.scales) + (size_t)l * SC_COUNT : nullptr;
    const uint16_t* h1 = at<uint16_t>(ws, L.h1);
    const uint16_t* qkv = at<uint16_t>(ws, L.qkv);
    const uint16_t* att = at<uint16_t>(ws, L.att);
    const uint16_t* h2 = at<uint16_t>(ws, L.h2);
    const uint16_t* act = at<uint16_t>(ws, L.act);
    if (f_back && l == D.L / 2 - 1) {  // the middle stream's share of the backout term
      ProfScope ps_(P_FEATURES, s);
      TRY(launch_axpy_stream(g, g_bf, gfin, W + P.backout(D), -1.f, Nd, s));
      g_amax_ok = false;
    }
    // ---- MLP ----
    if (f8) TRY(quant_dy(g_bf, d, sc + SC_G_MLP, g_amax_ok ? N : 0));
    {
      GemmArgs a;  // du = (g Wproj) * 2 relu(u)  with relu(u) = sqrt(act)
      ProfScope ps_(P_PROJ_DGRAD, s);
      a.M = N; a.N = hid; a.K = d;
      a.A = g_bf; a.lda = d; a.B = W + P.proj(D, l); a.ldb = hid; a.b_kcontig = 0;
      a.C = du; a.ldc = hid; a.aux = act; a.ldaux = hid;
      a.amax = qpart;  // NULL for bf16
      du_slots = f8 ? gemm_amax_slots(a) : 0;
      if (f8) TRY(dgrad_fp8(a, EPI_DRELU2, d, hid, at<uint8_t>(ws, L.wproj8), sc + SC_G_MLP, sc + SC_WPROJ));
      else TRY(gemm_bf16(a, EPI_DRELU2, s));
    }
    {
      ProfScope ps_(P_PROJ_WGRAD, s);  // dWproj = g^T act
      if (f8) TRY(wgrad_fp8(dyq, at<uint8_t>(ws, L.actq), sc + SC_G_MLP, sc + SC_ACT, G + P.proj(D, l), d, hid, N, acc, wpart, s));
      else TRY(wgrad(g_bf, d, act, hid, G + P.proj(D, l), d, hid, N, acc, wpart, s));
    }
    if (f8) TRY(quant_dy(du, hid, sc + SC_DU, du_slots));
    {
      GemmArgs a;  // dh = du Wfc (bf16)
      ProfScope ps_(P_FC_DGRAD, s);
      a.M = N; a.N = d; a.K = hid;
      a.A = du; a.lda = hid; a.B = W + P.fc(D, l); a.ldb = d; a.b_kcontig = 0;
      a.C = dh16; a.ldc = d;
      if (f8) TRY(dgrad_fp8(a, EPI_BF16, hid, d, at<uint8_t>(ws, L.wfc8), sc + SC_DU, sc + SC_WFC));
      else TRY(gemm_bf16(a, EPI_BF16, s));
    }
    {
      ProfScope ps_(P_FC_WGRAD, s);  // dWfc = du^T h2
      if (f8) TRY(wgrad_fp8(dyq, at<uint8_t>(ws, L.h2q), sc + SC_DU, sc + SC_H2, G + P.fc(D, l), hid, d, N, acc, wpart, s));
      else TRY(wgrad(du, hid, h2, d, G + P.fc(D, l), hid, d, N, acc, wpart, s));
    }
    { ProfScope ps_(P_RMSNORM_BWD, s); TRY(launch_rmsnorm_bwd(dh16, true, h2, at<float>(ws, L.r2), g, g_bf, N, d, s, qpart)); }
    // ---- attention ----
    if (f8) TRY(quant_dy(g_bf, d, sc + SC_G_ATT, N));
    {
      GemmArgs a;  // dO = g Wo
      ProfScope ps_(P_O_DGRAD, s);
      a.M = N; a.N = d; a.K = d;
      a.A = g_bf; a.lda = d; a.B = W + P.wo(D, l); a.ldb = d; a.b_kcontig = 0;
      a.C = dout; a.ldc = d;
      if (f8) TRY(dgrad_fp8(a, EPI_BF16, d, d, at<uint8_t>(ws, L.wo8), sc + SC_G_ATT, sc + SC_WO));
      else TRY(gemm_bf16(a, EPI_BF16, s));
    }
    {
      ProfScope ps_(P_O_WGRAD, s);  // dWo = g^T att
      if (f8) TRY(wgrad_fp8(dyq, at<uint8_t>(ws, L.attq), sc + SC_G_ATT, sc + SC_ATT, G + P.wo(D, l), d, d, N, acc, wpart, s));
      else TRY(wgrad(g_bf, d, att, d, G + P.wo(D, l), d, d, N, acc, wpart, s));
    }
    // dQ (and delta), then dK/dV; both leave through the QK-norm + rotary
    // backward into dqkv (bf16): the gradients of the raw q, k heads, and dv
    // (fp8: with the per-wave amax partials of dqkv)
    const QkNormBwd fuse{at<float>(ws, L.rq), at<float>(ws, L.rk), cs, dqkv, qpart};
    for (int part = 0; part < 2; ++part) {
      ProfScope ps_(part == 0 ? P_ATTN_BWD_Q : P_ATTN_BWD_KV, s);
      TRY(launch_attn_bwd_part(part, qkv, qkv + d, qkv + d + D.dkv, D.dqkv, att, dout, d, at<float>(ws, L.lse),
                               at<float>(ws, w.delta), nullptr, dqkv + d, dqkv + d + D.dkv, D.dqkv, D.B, D.H, D.Hkv,
                               D.T, D.layer_window(l), s, &fuse));
    }
    if (D.ve_layer(l)) {  // value embedding: dVE[token] += gate dv; gate-logit gradients dz
      ProfScope ps_(P_FEATURES, s);
      // per-token contributions gate dv (fp32, in du's memory: du is dead once the
      // MLP weight gradients are done, and holds 2 N 4d >= 4 N dkv bytes), then
      // each table row sums its tokens' contributions in token order
      float* vec = reinterpret_cast<float*>(du);
      TRY(launch_ve_bwd(ids, dqkv + d + D.dkv, D.dqkv, W + P.ve(D, l), at<float>(ws, L.vgate), vec, dzve, D.B, D.T,
                        D.Hkv, D.V, s));
      TRY(launch_embed_gather(vec, G + P.ve(D, l), (long long)N, D.dkv, D.V, true, at<void>(ws, w.emb), s));
    }
    if (f8) TRY(quant_dy(dqkv, D.dqkv, sc + SC_DQKV, attn_bwd_amax_slots(D.B, D.H, D.Hkv, D.T)));
    {
      GemmArgs a;  // dh = dqkv [Wq; Wk; Wv] (bf16)
      ProfScope ps_(P_QKV_DGRAD, s);
      a.M = N; a.N = d; a.K = D.dqkv;
      a.A = dqkv; a.lda = D.dqkv; a.B = W + P.qkv(D, l); a.ldb = d; a.b_kcontig = 0;
      a.C = dh16; a.ldc = d;
      if (f8) TRY(dgrad_fp8(a, EPI_BF16, D.dqkv, d, at<uint8_t>(ws, L.wqkv8), sc + SC_DQKV, sc + SC_WQKV));
      else TRY(gemm_bf16(a, EPI_BF16, s));
    }
    {
      ProfScope ps_(P_QKV_WGRAD, s);  // dWqkv = dqkv^T h1
      if (f8) TRY(wgrad_fp8(dyq, at<uint8_t>(ws, L.h1q), sc + SC_DQKV, sc + SC_H1, G + P.qkv(D, l), D.dqkv, d, N, acc, wpart, s));
      else TRY(wgrad(dqkv, D.dqkv, h1, d, G + P.qkv(D, l), D.dqkv, d, N, acc, wpart, s));
    }
    if (D.ve_layer(l)) {  // the gate reads h1[:, :32]: dh[:, :32] += dz Wg; dWg = dz^T h1[:, :32]
      ProfScope ps_(P_FEATURES, s);
      TRY(launch_ve_dh(dzve, W + P.vg(D, l), dh16, d, N, D.Hkv, s));
      TRY(launch_ve_gate_grad(dzve, h1, d, N, D.Hkv, fpart, G + P.vg(D, l), acc, s));
    }
    { ProfScope ps_(P_RMSNORM_BWD, s); TRY(launch_rmsnorm_bwd(dh16, true, h1, at<float>(ws, L.r1), g, g_bf, N, d, s, qpart)); }
    g_amax_ok = true;
    if (f_resid) {  // x' = resid_l x_in + x0lam_l x0
      ProfScope ps_(P_FEATURES, s);
      TRY(launch_resid_bwd(g, g_bf, at<uint16_t>(ws, L.xin), at<float>(ws, w.x0), g0, l == D.L - 1,
                           W + P.resid_l(l), W + P.x0lam(D, l), Nd, fpart, G + P.resid_l(l), G + P.x0lam(D, l), acc,
                           s));
      g_amax_ok = false;
    }
  }
  const float* gemb = g;
  if (f_smear || f_resid) {  // gradient of the embeddings: g + g0 through the smear backward (into dh)
    ProfScope ps_(P_FEATURES, s);
    TRY(launch_smear_bwd(ids, W + P.wte, f_smear ? W + P.smear_w(D) : nullptr, f_smear ? W + P.smear_lam(D) : nullptr,
                         g, g0, at<float>(ws, w.sig), dh, fpart, G + P.smear_lam(D), G + P.smear_w(D), acc, D.B, D.T,
                         d, D.V, s));
    gemb = dh;
  }
  {  // writes every row of the embedding gradient (adds to it when accumulating)
    ProfScope ps_(P_EMBED_BWD, s);
    if (!D.has(GPT_FEAT_VALUE_EMBED)) TRY(launch_embed_sort(ids, D.B, D.T, D.V, at<void>(ws, w.emb), s));
    TRY(launch_embed_gather(gemb, G + P.wte, N, d, D.V, acc, at<void>(ws, w.emb), s));
  }
  return GPT_OK;
}

// ---------------------------------------------------------------------------
// AdamW
// ---------------------------------------------------------------------------
extern "C" gpt_status adamw_update(float* W, uint16_t* W_bf16, const float* G, float* M, float* V, size_t n,
                                   int32_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                                   float grad_scale, gpt_stream_t stream) {
  if (n == 0) return GPT_OK;
  if (!W || !G || !M || !V) FAIL(GPT_ERR_INVALID_ARG, "W, G, M and V must not be NULL");
  if (n % 4) FAIL(GPT_ERR_INVALID_ARG, "n must be a multiple of 4");
  if (((uintptr_t)W | (uintptr_t)G | (uintptr_t)M | (uintptr_t)V) & 15) FAIL(GPT_ERR_INVALID_ARG, "fp32 arrays must be 16-byte aligned");
  if ((uintptr_t)W_bf16 & 7) FAIL(GPT_ERR_INVALID_ARG, "W_bf16 must be 8-byte aligned");
  if (step < 1) FAIL(GPT_ERR_INVALID_ARG, "step is 1-based");
  if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) || !(eps > 0.f))
    FAIL(GPT_ERR_INVALID_ARG, "need 0 <= beta1, beta2 < 1 and eps > 0");
  const double bc1 = 1.0 - pow((double)beta1, (double)step), bc2 = 1.0 - pow((double)beta2, (double)step);
  ProfScope ps_(P_ADAMW, S(stream));
  TRY(launch_adamw(W, W_bf16, G, M, V, (long long)n, lr, beta1, beta2, eps, weight_decay, (float)(1.0 / bc1),
                   (float)(1.0 / bc2), grad_scale, S(stream)));
  return GPT_OK;
}

// ---------------------------------------------------------------------------
// Muon
// ---------------------------------------------------------------------------
namespace {

constexpr int kFrobBlocks = 64;

struct MuonWS {
  size_t partial, Xb0, Xb1, Ab, Bb, gpart, nm_part, nm_scale, total;
};

// The Gram product A = X^T X of a Newton-Schulz iteration: k-split count and
// whether only the tiles on and above the diagonal are computed (then
// mirrored).  Symmetric when the batch holds more 128 x 128 tiles than the
// chip has CUs, or when K is split: the split multiplies the workgroups, so
// halving the tiles lets about twice as many splits share a grid (one
// 1664 x 6656 matrix: 91 tiles x 6 splits instead of 169 x 4).
struct GramPlan {
  int splits, sym;
};
inline GramPlan gram_plan(int count, int rows, int cols) {
  const int lrow = std::max(rows, cols), sm = std::min(rows, cols);
  const long long t = (sm + 127) / 128;
  const long long full = (long long)count * t * t, upper = (long long)count * t * (t + 1) / 2;
  if (full >= 512 || lrow / 1024 <= 1) return {1, full > 256 ? 1 : 0};
  const long long tiles = full > 256 ? full : upper;  // the symmetric grid when the split applies
  const int splits = (int)std::max<long long>(1, std::min<long long>(lrow / 1024, (512 + tiles - 1) / tiles));
  return {splits, (splits > 1 || full > 256) ? 1 : 0};
}

MuonWS muon_layout(int count, int rows, int cols) {
  MuonWS m;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = al(o + bytes); return r; };
  const size_t n = (size_t)count * rows * cols;
  const size_t sm = (size_t)std::min(rows, cols);
  m.partial = take((size_t)count * kFrobBlocks * 4);
  m.Xb0 = take(n * 2);
  m.Xb1 = take(n * 2);
  m.Ab = take((size_t)count * sm * sm * 2);
  m.Bb = take((size_t)count * sm * sm * 2);
  const int gs_ = gram_plan(count, rows, cols).splits;
  m.gpart = take(gs_ > 1 ? (size_t)gs_ * count * sm * sm * 4 : 4);
  m.nm_part = take((size_t)normuon_part_floats(count, rows, cols) * 4);
  m.nm_scale = take((size_t)count * std::max(rows, cols) * 4);
  m.total = o;
  return m;
}

int check_muon_shape(int32_t count, int32_t rows, int32_t cols) {
  if (count < 1 || rows < 1 || cols < 1) FAIL(GPT_ERR_INVALID_ARG, "count, rows and cols must be >= 1");
  if ((rows % 8) || (cols % 8)) FAIL(GPT_ERR_INVALID_ARG, "rows and cols must be multiples of 8");
  if ((long long)rows * cols > (1LL << 30) || (long long)count * rows * cols > (1LL << 34))
    FAIL(GPT_ERR_INVALID_ARG, "matrices too large");
  return 0;
}

}  // namespace

extern "C" gpt_status muon_workspace_size(int32_t count, int32_t rows, int32_t cols, size_t* bytes) {
  TRY(check_muon_shape(count, rows, cols));
  if (!bytes) FAIL(GPT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = muon_layout(count, rows, cols).total;
  return GPT_OK;
}

namespace {
struct NorMuonArgs {
  float* V;
  int per_row;
  float beta2, eps;
};

int muon_impl(float* Wt, uint16_t* W_bf16, const float* Gm, float* M, float* O_out, int32_t count, int32_t rows,
              int32_t cols, const float* coeffs, int32_t ns_steps, float lr, float momentum, float weight_decay,
              const NorMuonArgs* nm, void* ws, size_t ws_bytes, gpt_stream_t stream) {
  TRY(check_muon_shape(count, rows, cols));
  if (!Gm) FAIL(GPT_ERR_INVALID_ARG, "G is NULL");
  if (!coeffs) FAIL(GPT_ERR_INVALID_ARG, "coeffs is NULL");
  if (ns_steps < 1 || ns_steps > 16) FAIL(GPT_ERR_INVALID_ARG, "ns_steps must be in [1, 16]");
  if (W_bf16 && !Wt) FAIL(GPT_ERR_INVALID_ARG, "W_bf16 given without W");
  if (!ws || ((uintptr_t)ws % kAlign)) FAIL(GPT_ERR_INVALID_ARG, "workspace NULL or not 256-byte aligned");
  if (((uintptr_t)Gm | (uintptr_t)M) & 15) FAIL(GPT_ERR_INVALID_ARG, "G and M must be 16-byte aligned");
  for (int i = 0; i < 3 * ns_steps; ++i)
    if (!isfinite(coeffs[i])) FAIL(GPT_ERR_INVALID_ARG, "non-finite coefficient");
  const MuonWS m = muon_layout(count, rows, cols);
  if (ws_bytes < m.total) FAIL(GPT_ERR_WORKSPACE, "workspace smaller than muon_workspace_size()");
  hipStream_t s = S(stream);
  const long long per = (long long)rows * cols;
  const int lrow = std::max(rows, cols), sm = std::min(rows, cols);

  const float* src = M ? M : Gm;
  float* partial = at<float>(ws, m.partial);
  uint16_t* Xb[2] = {at<uint16_t>(ws, m.Xb0), at<uint16_t>(ws, m.Xb1)};
  uint16_t* Ab = at<uint16_t>(ws, m.Ab);
  uint16_t* Bb = at<uint16_t>(ws, m.Bb);
  {  // M <- momentum M + G with the Frobenius partials of the new M, or the partials of G alone
    ProfScope ps_(P_MUON_ELEMWISE, s);
    if (M) TRY(launch_momentum_frob(M, Gm, momentum, partial, count, per, kFrobBlocks, s));
    else TRY(launch_frob_partial(src, partial, count, per, kFrobBlocks, s));
  }
  { ProfScope ps_(P_MUON_ELEMWISE, s); TRY(launch_ns_init(src, partial, kFrobBlocks, nullptr, Xb[0], count, rows, cols, 1e-7f, s)); }

  const long long sX = (long long)lrow * sm, sA = (long long)sm * sm;
  const GramPlan gplan = gram_plan(count, rows, cols);
  const int gram_split = gplan.splits;
  float* gpart = at<float>(ws, m.gpart);
  int cur = 0;
  // A = X^T X and B = b A + c A A are symmetric: when the batch holds more
  // 128 x 128 tiles than the chip has CUs, both products compute only the
  // tiles on and above the diagonal, and their bf16 outputs, which the next
  // product reads in full, are mirrored (with fewer tiles all of them run in
  // one wave anyway, and the mirror would only add time; the Gram product
  // also when its K is split, see gram_plan).  A is kept in bf16
  // only, like the iteration's other operands: the polynomial's epilogue
  // reads the same bf16 A its product reads (the b A term then carries one
  // bf16 rounding, as B itself does when it is stored).
  const long long t128 = (sm + 127) / 128;
  const int sym = (long long)count * t128 * t128 > 256 ? 1 : 0;  // the polynomial product
  const int gsym = gplan.sym;
  GemmArgs ga;
  ga.M = sm; ga.N = sm; ga.K = lrow; ga.batch = count; ga.sym = gsym;
  ga.lda = sm; ga.sA = sX; ga.a_kcontig = 0;
  ga.ldb = sm; ga.sB = sX; ga.b_kcontig = 0;
  ga.C = Ab; ga.ldc = sm; ga.sC = sA;
  if (gram_split > 1) {
    // split-K partials [split][count][sm][sm], then Ab = bf16(sum)
    ga.C = gpart; ga.k_split = gram_split; ga.split_stride = sA * count;
  }
  GemmArgs gp;
  gp.M = sm; gp.N = sm; gp.K = sm; gp.batch = count; gp.sym = sym;
  gp.A = Ab; gp.lda = sm; gp.sA = sA;
  gp.B = Ab; gp.ldb = sm; gp.sB = sA; gp.b_kcontig = 0;
  gp.C = Bb; gp.ldc = sm; gp.sC = sA;
  gp.aux = Ab; gp.ldaux = sm; gp.sAux = sA;
  for (int it = 0; it < ns_steps; ++it) {
    const float ca = coeffs[3 * it], cb = coeffs[3 * it + 1], cc = coeffs[3 * it + 2];
    {
      ProfScope ps_(P_NS_GRAM, s);
      GemmArgs a = ga;  // A = X^T X (bf16)
      a.A = Xb[cur]; a.B = Xb[cur];
      if (gram_split <= 1) {
        TRY(gemm_bf16(a, EPI_BF16, s));
      } else {
        TRY(gemm_bf16(a, EPI_F32, s));
        TRY(launch_splitk_reduce(gpart, gram_split, sA * count, nullptr, Ab, sA * count, 0.f, s));
      }
      if (gsym) TRY(launch_sym_mirror(Ab, sm, sm, sA, count, s));
    }
    {
      ProfScope ps_(P_NS_POLY, s);
      GemmArgs a = gp;  // B = b A + c A A
      a.alpha = cc; a.beta = cb;
      TRY(gemm_bf16(a, EPI_NS_POLY, s));
      if (sym) TRY(launch_sym_mirror(Bb, sm, sm, sA, count, s));
    }
    {
      // X = a X + X B, X kept in bf16 (as the iteration's products read it;
      // the orthogonalised update leaves in bf16): the polynomial's epilogue
      // form, beta X + (X B)
      GemmArgs a;
      ProfScope ps_(P_NS_UPDATE, s);
      a.M = lrow; a.N = sm; a.K = sm; a.batch = count;
      a.A = Xb[cur]; a.lda = sm; a.sA = sX;
      a.B = Bb; a.ldb = sm; a.sB = sA; a.b_kcontig = 0;
      a.aux = Xb[cur]; a.ldaux = sm; a.sAux = sX;
      a.beta = ca;
      a.C = Xb[cur ^ 1]; a.ldc = sm; a.sC = sX;
      TRY(gemm_bf16(a, EPI_NS_POLY, s));
    }
    cur ^= 1;
  }
  const uint16_t* X = Xb[cur];  // the last update's output
  const float* nsc = nullptr;
  if (nm) {
    ProfScope ps_(P_MUON_ELEMWISE, s);
    float* scale = at<float>(ws, m.nm_scale);
    TRY(launch_normuon_scale(X, at<float>(ws, m.nm_part), nm->V, scale, count, rows, cols, nm->per_row, nm->beta2,
                             nm->eps, s));
    nsc = scale;
  }
  {
    ProfScope ps_(P_MUON_ELEMWISE, s);
    TRY(launch_muon_apply(X, Wt, W_bf16, O_out, count, rows, cols, lr, weight_decay, nsc, nm ? nm->per_row : 0, s));
  }
  return GPT_OK;
}
}  // namespace

extern "C" gpt_status muon_update(float* Wt, uint16_t* W_bf16, const float* Gm, float* M, float* O_out,
                                  int32_t count, int32_t rows, int32_t cols, const float* coeffs,
                                  int32_t ns_steps, float lr, float momentum, float weight_decay, void* ws,
                                  size_t ws_bytes, gpt_stream_t stream) {
  return (gpt_status)muon_impl(Wt, W_bf16, Gm, M, O_out, count, rows, cols, coeffs, ns_steps, lr, momentum, weight_decay,
                   nullptr, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Muon without any allocation: the workspace is a file-scope device array
// ---------------------------------------------------------------------------
// Every GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in): the device address of this GPU's copy comes
// from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[GPT_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_ptr(void** out) {
  int dev = 0;
  GS_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) FAIL(GPT_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    GS_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || ((uintptr_t)p % kAlign)) FAIL(GPT_ERR_HIP, "scratch symbol address missing or misaligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}
}  // namespace

extern "C" gpt_status muon_update_noalloc(float* Wt, uint16_t* W_bf16, const float* Gm, float* M, float* O_out,
                                          int32_t count, int32_t rows, int32_t cols, const float* coeffs,
                                          int32_t ns_steps, float lr, float momentum, float weight_decay,
                                          gpt_stream_t stream) {
  TRY(check_muon_shape(count, rows, cols));
  const size_t need = muon_layout(count, rows, cols).total;
  if (need > (size_t)GPT_NOALLOC_SCRATCH_BYTES)
    FAIL(GPT_ERR_WORKSPACE, "muon_update_noalloc: these matrices need " + std::to_string(need) +
                                " bytes of scratch, more than the " + std::to_string((size_t)GPT_NOALLOC_SCRATCH_BYTES) +
                                " the library holds per GPU; call muon_update with a workspace");
  void* ws = nullptr;
  TRY(scratch_ptr(&ws));
  return (gpt_status)muon_impl(Wt, W_bf16, Gm, M, O_out, count, rows, cols, coeffs, ns_steps, lr, momentum,
                               weight_decay, nullptr, ws, (size_t)GPT_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" gpt_status normuon_update(float* Wt, uint16_t* W_bf16, const float* Gm, float* M, float* V,
                                     float* O_out, int32_t count, int32_t rows, int32_t cols, int32_t per_row,
                                     const float* coeffs, int32_t ns_steps, float lr, float momentum,
                                     float weight_decay, float beta2, float eps, void* ws, size_t ws_bytes,
                                     gpt_stream_t stream) {
  if (!V) FAIL(GPT_ERR_INVALID_ARG, "V (the per-neuron second moments) is NULL");
  if (per_row != 0 && per_row != 1) FAIL(GPT_ERR_INVALID_ARG, "per_row must be 0 or 1");
  if (!(beta2 >= 0.f && beta2 < 1.f)) FAIL(GPT_ERR_INVALID_ARG, "beta2 must be in [0, 1)");
  if (!(eps >= 0.f) || !isfinite(eps)) FAIL(GPT_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const NorMuonArgs nm{V, per_row, beta2, eps};
  return (gpt_status)muon_impl(Wt, W_bf16, Gm, M, O_out, count, rows, cols, coeffs, ns_steps, lr, momentum, weight_decay, &nm,
                   ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// component: attention
// ---------------------------------------------------------------------------
namespace {
int check_attn(int32_t batch, int32_t n_head, int32_t n_kv_head, int32_t seq_len) {
  if (batch < 0 || n_head < 1 || seq_len < 0) FAIL(GPT_ERR_INVALID_ARG, "bad batch/n_head/seq_len");
  if (n_kv_head < 1 || n_head % n_kv_head) FAIL(GPT_ERR_INVALID_ARG, "n_kv_head must divide n_head");
  return 0;
}
}  // namespace

extern "C" gpt_status gpt_op_attention_fwd(int32_t batch, int32_t n_head, int32_t n_kv_head, int32_t seq_len,
                                           int32_t window, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                           int64_t ld_qkv, uint16_t* out, int64_t ld_out, float* lse,
                                           gpt_stream_t stream) {
  TRY(check_attn(batch, n_head, n_kv_head, seq_len));
  if (batch == 0 || seq_len == 0) return GPT_OK;
  if (!q || !k || !v || !out || !lse) FAIL(GPT_ERR_INVALID_ARG, "NULL pointer");
  if (ld_qkv < (int64_t)n_head * 128 || ld_out < (int64_t)n_head * 128 || (ld_qkv % 8) || (ld_out % 8))
    FAIL(GPT_ERR_INVALID_ARG, "leading dimensions must be >= 128*n_head and multiples of 8");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) FAIL(GPT_ERR_INVALID_ARG, "misaligned");
  TRY(launch_attn_fwd(q, k, v, ld_qkv, out, ld_out, lse, batch, n_head, n_kv_head, seq_len, window < 0 ? -1 : window,
                      S(stream)));
  return GPT_OK;
}

extern "C" gpt_status gpt_op_attention_bwd(int32_t batch, int32_t n_head, int32_t n_kv_head, int32_t seq_len,
                                           int32_t window, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                           int64_t ld_qkv, const uint16_t* out, const uint16_t* dout, int64_t ld_out,
                                           const float* lse, float* delta, float* dq_acc, uint16_t* dk, uint16_t* dv,
                                           int64_t ld_dkv, gpt_stream_t stream) {
  TRY(check_attn(batch, n_head, n_kv_head, seq_len));
  if (batch == 0 || seq_len == 0) return GPT_OK;
  if (!q || !k || !v || !out || !dout || !lse || !delta || !dq_acc || !dk || !dv)
    FAIL(GPT_ERR_INVALID_ARG, "NULL pointer");
  if (ld_qkv < (int64_t)n_kv_head * 128 || ld_out < (int64_t)n_head * 128 || ld_dkv < (int64_t)n_kv_head * 128 ||
      (ld_qkv % 8) || (ld_out % 8) || (ld_dkv % 8))
    FAIL(GPT_ERR_INVALID_ARG, "leading dimensions too small or not multiples of 8");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dk |
       (uintptr_t)dv | (uintptr_t)dq_acc) & 15)
    FAIL(GPT_ERR_INVALID_ARG, "misaligned");
  TRY(launch_attn_bwd(q, k, v, ld_qkv, out, dout, ld_out, lse, delta, dq_acc, dk, dv, ld_dkv, batch, n_head, n_kv_head,
                      seq_len, window < 0 ? -1 : window, S(stream)));
  return GPT_OK;
}

// ---------------------------------------------------------------------------
// roofline probe
// ---------------------------------------------------------------------------
extern "C" gpt_status gpt_probe_mfma(int32_t fp8, int32_t blocks, int32_t iters, float* out, double* flops,
                                     gpt_stream_t stream) {
  if (blocks < 1 || iters < 1 || !out || !flops) FAIL(GPT_ERR_INVALID_ARG, "bad probe arguments");
  TRY(launch_mfma_peak(fp8 ? 1 : 0, blocks, iters, out, flops, S(stream)));
  return GPT_OK;
}
