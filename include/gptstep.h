/*
 * gptstep.h -- C ABI of libgptstep.so: one pretraining step of a depth-
 * parameterised decoder-only GPT (forward, backward, Muon update) on AMD
 * MI355X (gfx950).
 *
 * What is computed follows the nanochat pages:
 *   dev.to, "¿Cómo Entrenar Tu Propio ChatGPT por $50?":
 *     "La Filosofía: Un Solo Selector" -- one dial, the depth;
 *     "1. Modelo GPT (nanochat/gpt.py)" -- RoPE, QK normalisation, untied
 *        embedding and head, ReLU^2 MLP, causal flash attention;
 *     "2. Optimizador Muon (nanochat/optim.py)" -- Newton-Schulz iteration
 *        A = X^T X, B = b A + c A A, X = a X + X B over a coefficient table;
 *     "3. Gestión de Precisión (nanochat/common.py)" -- fp32 master weights,
 *        weights cast to the bf16 compute dtype for each matmul;
 *   apidog.com/pt and apidog.com/de, the precision sections -- the fp8 option
 *     with one scale per tensor ("escalonamento por tensor", "tensorweise").
 *
 * Shapes come from the depth alone: d_model = 64 * depth, heads of width 128
 * (so n_head = d_model / 128 and depth must be even), MLP hidden = 4 * d_model.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the comment says "host".
 *   - The caller owns all memory.  The library never allocates or frees
 *     device memory; scratch space comes from a caller-provided workspace
 *     whose size is queried first (muon_update_noalloc alone uses a device
 *     array the library holds instead).
 *   - Every call validates its arguments on the host first and returns a
 *     status; no argument error ever reaches the device.  Kernel launch
 *     failures return GPT_ERR_HIP with details in gpt_last_error().
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  No call synchronises the device; results (including
 *     the loss) are in device memory when the stream reaches them.
 *   - Token ids belong in [0, vocab).  An id outside that range is never
 *     used as an index: its embedding (and value-embedding) rows are taken
 *     as zero and it adds nothing to any gradient; the loss of a position
 *     whose target is outside the range is undefined.
 *   - Preconditions that are not checked (they would need a device sync):
 *     device buffers of the stated sizes;
 *     gpt_step_bwd follows gpt_step_fwd on the same stream with the same
 *     shape, parameters, ids and workspace, with no other use of that
 *     workspace in between.
 *   - Not thread-safe across calls that share a workspace or outputs.
 */
#ifndef GPTSTEP_H
#define GPTSTEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* gpt_stream_t; /* hipStream_t */

typedef enum {
  GPT_OK = 0,
  GPT_ERR_INVALID_ARG = -1, /* null required pointer, bad count/size/flag */
  GPT_ERR_SHAPE = -2,       /* depth odd or < 2, vocab/seq_len/batch < 1, too large */
  GPT_ERR_WORKSPACE = -3,   /* workspace smaller than the queried size */
  GPT_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  GPT_ERR_UNSUPPORTED = -5  /* unknown precision or layout */
} gpt_status;

typedef enum {
  GPT_PREC_BF16 = 0, /* bf16 operands, fp32 accumulation */
  GPT_PREC_FP8 = 1   /* the four block GEMMs in fp8 (E4M3 activations and
                        weights, E5M2 output gradients, one fp32 scale per
                        tensor); head, attention and Muon stay bf16 */
} gpt_precision;

/* The model and batch.  d_model = 64*depth, n_head = d_model/128,
 * hidden = 4*d_model.  Limits: 2 <= depth <= 64 and even; 1 <= vocab <= 2^24;
 * 1 <= seq_len <= 16384; 1 <= batch; batch*seq_len <= 2^24.
 *
 * Attention variants (dev.to page, "1. Modelo GPT": grouped-query attention
 * and sliding-window layers in a pattern such as "SSSL"; "5. Unificación Flash
 * Attention": the window_size argument).  Zero-initialised fields give plain
 * multi-head, full causal attention in every layer:
 *   n_kv_head       key/value heads (0 = n_head); must divide n_head.  Query
 *                   head h reads key/value head h / (n_head / n_kv_head).
 *   window          left window of the short layers: query i sees keys
 *                   i - window .. i (0 = no short layers).
 *   pattern_len     length of the layer pattern, 1 .. 32 (0 = all long);
 *   pattern_long    bit i set = pattern position i is 'L' (full causal),
 *                   clear = 'S' (windowed); layer l takes position l % len.
 *                   "SSSL" is pattern_len 4, pattern_long 0x8. */
/* Record-model features (the same model section: value embeddings in the
 * ResFormer style; the efficiency tricks per-layer residual scaling, smear and
 * backout), bits of gpt_shape.features:
 *   GPT_FEAT_VALUE_EMBED  layers 0, 2, 4, ... add to v, per key/value head,
 *                         gate * VE_l[token] with gate = 3 sigmoid(h[:32] .
 *                         Wg_l[head]), h the attention input (normed stream)
 *   GPT_FEAT_SMEAR        token t >= 1 adds lam sigmoid(e_t[:24] . w) e_{t-1}
 *                         to its embedding e_t (within its sequence)
 *   GPT_FEAT_RESID_LAMBDA layer l starts with x <- resid_l x + x0lam_l x0, x0
 *                         the stream after the embedding (and smear)
 *   GPT_FEAT_BACKOUT      before the final norm x <- x - backout x_mid, x_mid
 *                         the stream after layer depth/2 - 1
 * With features != 0 the packed parameters gain, after lm_head: VE_l [V, dkv]
 * for l = 0, 2, ..; Wg_l [n_kv_head, 32] for the same l; then the scalar block
 * resid [depth], x0lam [depth], w [24], lam [1], backout [1], 6 unused.
 * Every one of them is present when any bit is set (a cleared bit leaves its
 * parameters unused, gradient 0).  Scalars are read on the device from the
 * bf16 copy, like every other parameter. */
enum {
  GPT_FEAT_VALUE_EMBED = 1,
  GPT_FEAT_SMEAR = 2,
  GPT_FEAT_RESID_LAMBDA = 4,
  GPT_FEAT_BACKOUT = 8
};

typedef struct {
  int32_t depth;
  int32_t vocab;
  int32_t seq_len;   /* T: tokens per sequence (ids carry T+1 per row) */
  int32_t batch;     /* B: sequences per step */
  int32_t precision; /* gpt_precision */
  int32_t n_kv_head;
  int32_t window;
  int32_t pattern_len;
  uint32_t pattern_long;
  uint32_t features; /* GPT_FEAT_* bits; 0 = the plain model */
} gpt_shape;

/* Packed parameter buffers, all with gpt_param_count() elements in the packed
 * order: wte [V,d] | for each layer: wq [d,d], wk [dkv,d], wv [dkv,d], wo [d,d]
 * (dkv = 128 n_kv_head; d without grouped heads) | for each layer wfc [4d,d] |
 * for each layer wproj [d,4d] | lm_head [V,d], each row-major [out, in].  wq,
 * wk, wv of one layer are adjacent, so they form one [d+2dkv, d] operand.
 * Without grouped heads the S group is the 4*depth [d,d] matrices; the F group
 * is the depth wfc matrices, the P group the depth wproj matrices. */
typedef struct {
  const float* master;  /* fp32 master weights (read by nothing in fwd/bwd) */
  const uint16_t* bf16; /* bf16 working copy (bit patterns) used by fwd/bwd */
  float* grad;          /* fp32 gradients, written by gpt_step_bwd */
} gpt_params;

/* Number of parameters (elements) of the packed buffers. */
gpt_status gpt_param_count(const gpt_shape* shape, size_t* n_params /* host */);

/* Element offsets of the 2 + 6*depth tensors in packed order (wte, then per
 * layer wq wk wv wo, then each wfc, then each wproj, then lm_head), followed
 * when gpt_shape.features != 0 by the depth/2 value-embedding tables, the
 * depth/2 gate matrices and the scalar block (resid, x0lam, w, lam, backout,
 * unused): 2 + 6*depth + depth + 6 tensors in all.
 * `offsets` (host) must hold `capacity` entries; *n_tensors (host) receives
 * the count.  GPT_ERR_INVALID_ARG when capacity is too small. */
gpt_status gpt_param_layout(const gpt_shape* shape, size_t* offsets, int32_t capacity,
                            int32_t* n_tensors);

/* Bytes of workspace that gpt_step_fwd / gpt_step_bwd need for this shape
 * (activations saved by the forward pass plus backward scratch). */
gpt_status gpt_workspace_size(const gpt_shape* shape, size_t* bytes /* host */);

/* dst[i] = bf16(src[i]), round to nearest even; n elements. */
gpt_status gpt_cast_bf16(const float* src, uint16_t* dst, size_t n, gpt_stream_t stream);

/* Forward pass and loss (dev.to page, "1. Modelo GPT"; the loss is the mean
 * cross-entropy of next-token prediction over all batch*seq_len positions).
 *   ids     int32 [batch, seq_len+1]; inputs ids[:, :T], targets ids[:, 1:].
 *   loss    fp32 [1]: mean loss.
 *   row_lse nullable fp32 [batch*seq_len]: log-sum-exp of each row's logits.
 *   logits  nullable fp32 [batch*seq_len, vocab]: full logits, meant for
 *           tiny shapes only (the normal path never forms them).
 *   ws      workspace of at least gpt_workspace_size() bytes, 256-aligned.
 * The workspace keeps the activations gpt_step_bwd needs. */
gpt_status gpt_step_fwd(const gpt_shape* shape, const gpt_params* params, const int32_t* ids,
                        float* loss, float* row_lse, float* logits, void* ws, size_t ws_bytes,
                        gpt_stream_t stream);

/* Backward pass of the mean loss: writes (accumulate = 0) or adds
 * (accumulate = 1) the gradient of every parameter into params->grad. */
gpt_status gpt_step_bwd(const gpt_shape* shape, const gpt_params* params, const int32_t* ids,
                        int32_t accumulate, void* ws, size_t ws_bytes, gpt_stream_t stream);

/* Backward of loss_scale * (sum of the B*T row losses) instead of the mean:
 * gpt_step_bwd is this call with loss_scale = 1/(batch*seq_len).  For a
 * batch split into n_micro micro-batches of the same shape, calling it on each
 * with loss_scale = 1/(n_micro*batch*seq_len), accumulate = 0 for the first
 * and 1 after, leaves the gradient of the mean loss over all of them (the
 * pages' gradient accumulation when one GPU stands in for several: dev.to
 * page, FAQ "¿Qué GPU necesito?").  loss_scale > 0 and finite. */
gpt_status gpt_step_bwd_scaled(const gpt_shape* shape, const gpt_params* params, const int32_t* ids,
                               int32_t accumulate, float loss_scale, void* ws, size_t ws_bytes,
                               gpt_stream_t stream);

/* AdamW with decoupled weight decay on n fp32 parameters, for the matrices
 * the pages give to AdamW (dev.to page, "2. Optimizador Muon": embeddings and
 * lm_head):
 *   g = grad_scale * G;  M <- beta1 M + (1-beta1) g;  V <- beta2 V + (1-beta2) g^2
 *   W <- W (1 - lr weight_decay) - lr (M / (1-beta1^step)) / (sqrt(V / (1-beta2^step)) + eps)
 *   W_bf16 <- bf16(W) (nullable)
 * step: 1-based count of this update (bias correction).  M and V start at 0.
 * n % 4 == 0; W, G, M, V 16-byte aligned, W_bf16 8-byte aligned.
 * GPT_ERR_INVALID_ARG for NULL arrays, step < 1, betas outside [0, 1), eps <= 0. */
gpt_status adamw_update(float* W, uint16_t* W_bf16, const float* G, float* M, float* V, size_t n, int32_t step,
                        float lr, float beta1, float beta2, float eps, float weight_decay, float grad_scale,
                        gpt_stream_t stream);

/* Workspace bytes for muon_update / normuon_update on `count` matrices of
 * [rows, cols]. */
gpt_status muon_workspace_size(int32_t count, int32_t rows, int32_t cols, size_t* bytes /* host */);

/* Muon update of `count` same-shape fp32 matrices [rows, cols], contiguous
 * (dev.to page, "2. Optimizador Muon"):
 *   M <- momentum * M + G                      (skipped when M is NULL: M := G)
 *   X <- M / (||M||_F + 1e-7), oriented so that rows >= cols
 *   for each (a, b, c) of coeffs[0 .. ns_steps-1]:
 *       A = X^T X;  B = b A + c A A;  X = a X + X B   (bf16 MFMA, fp32 accumulate,
 *                                                      X kept in fp32)
 *   O = X oriented back to [rows, cols]
 *   W <- W * (1 - lr * weight_decay) - lr * O;  W_bf16 <- bf16(W)
 * W, W_bf16 and O_out are each nullable (W NULL: no apply; O_out: copy of O).
 * coeffs: HOST array of 3*ns_steps floats (a, b, c per iteration);
 * 1 <= ns_steps <= 16.  G may alias M only when M is NULL. */
gpt_status muon_update(float* W, uint16_t* W_bf16, const float* G, float* M, float* O_out,
                       int32_t count, int32_t rows, int32_t cols, const float* coeffs,
                       int32_t ns_steps, float lr, float momentum, float weight_decay, void* ws,
                       size_t ws_bytes, gpt_stream_t stream);

/* Muon with the NorMuon per-neuron rescale (dev.to page, "2. Optimizador
 * Muon", NorMuon variance reduction; apidog.com/pt "Redução de Variância
 * NorMuon"): as muon_update, with O replaced before the apply by
 *   vm_i   = mean of O_i^2 over neuron i's weights
 *   V_i   <- beta2 * V_i + (1 - beta2) * vm_i        (V = 0 before step 1)
 *   step_i = 1 / (sqrt(V_i) + eps)
 *   O_i   <- O_i * step_i * sqrt(sum vm) / max(sqrt(sum vm step^2), 1e-10)
 * (sums over the neurons of one matrix).  A neuron is a row of W when
 * per_row = 1 (the statistic runs over the inputs), a column when 0.
 * V: device fp32 [count, rows] (per_row) or [count, cols], updated in place.
 * O_out receives the rescaled O.  Workspace: muon_workspace_size.
 * GPT_ERR_INVALID_ARG for V NULL, per_row not 0/1, beta2 outside [0, 1),
 * eps negative or not finite, and everything muon_update rejects. */
gpt_status normuon_update(float* W, uint16_t* W_bf16, const float* G, float* M, float* V, float* O_out,
                          int32_t count, int32_t rows, int32_t cols, int32_t per_row, const float* coeffs,
                          int32_t ns_steps, float lr, float momentum, float weight_decay, float beta2, float eps,
                          void* ws, size_t ws_bytes, gpt_stream_t stream);

/* muon_update for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments and results as muon_update, without the workspace
 * arguments.  Its scratch space is a device array the library holds on each
 * GPU it runs on, GPT_NOALLOC_SCRATCH_BYTES bytes, until the process ends;
 * the call makes no allocation of any kind.  Shapes whose
 * muon_workspace_size() exceeds that size return GPT_ERR_WORKSPACE (the
 * message names both sizes).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (different streams, or threads) race, and
 * must be ordered by the caller.  Nothing in the array needs to be cleared
 * between calls.  GPT_ERR_HIP if the array's device address cannot be
 * taken. */
#define GPT_NOALLOC_SCRATCH_BYTES (160u * 1024u * 1024u)
gpt_status muon_update_noalloc(float* W, uint16_t* W_bf16, const float* G, float* M, float* O_out,
                               int32_t count, int32_t rows, int32_t cols, const float* coeffs,
                               int32_t ns_steps, float lr, float momentum, float weight_decay,
                               gpt_stream_t stream);

/* Text of a status, and the message of the last failing call on this thread
 * (empty when none).  Both return static or thread-local storage. */
const char* gpt_status_string(gpt_status status);
const char* gpt_last_error(void);

/* Library ABI version (bumped on any signature change; 2: gpt_shape carries
 * the attention variants; 3: gpt_shape.features). */
int32_t gpt_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GPTSTEP_H */
