"""ctypes binding of libgptstep.so (argument marshalling only).

Every function here converts torch tensors to device pointers, picks the
current HIP stream and calls the C entry point of the same name; all compute
runs in the library's HIP kernels.  A missing library raises at import: there
is no fallback path.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgptstep.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m gpt_transformer_step_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

PREC_BF16, PREC_FP8 = 0, 1
LAYOUT_K, LAYOUT_MN = 0, 1
DTYPE_F32, DTYPE_BF16 = 0, 1
FP8_E4M3, FP8_E5M2 = 0, 1

STATUS = {0: "ok", -1: "invalid argument", -2: "invalid shape", -3: "workspace too small",
          -4: "HIP runtime error", -5: "unsupported"}


class GptError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn}: {STATUS.get(code, code)} ({code}): {msg}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("depth", ctypes.c_int32), ("vocab", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("precision", ctypes.c_int32), ("n_kv_head", ctypes.c_int32),
                ("window", ctypes.c_int32), ("pattern_len", ctypes.c_int32), ("pattern_long", ctypes.c_uint32),
                ("features", ctypes.c_uint32)]


# record-model feature letters -> gpt_shape.features bits
FEATURE_BITS = {"v": 1, "s": 2, "r": 4, "b": 8}


class Params(ctypes.Structure):
    _fields_ = [("master", ctypes.c_void_p), ("bf16", ctypes.c_void_p), ("grad", ctypes.c_void_p)]


_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_P = ctypes.POINTER

_SIGS = {
    "gpt_param_count": [_P(Shape), _P(_sz)],
    "gpt_param_layout": [_P(Shape), _P(_sz), _i32, _P(_i32)],
    "gpt_workspace_size": [_P(Shape), _P(_sz)],
    "gpt_cast_bf16": [_vp, _vp, _sz, _vp],
    "gpt_step_fwd": [_P(Shape), _P(Params), _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "gpt_step_bwd": [_P(Shape), _P(Params), _vp, _i32, _vp, _sz, _vp],
    "gpt_step_bwd_scaled": [_P(Shape), _P(Params), _vp, _i32, _f32, _vp, _sz, _vp],
    "adamw_update": [_vp, _vp, _vp, _vp, _vp, _sz, _i32, _f32, _f32, _f32, _f32, _f32, _f32, _vp],
    "muon_workspace_size": [_i32, _i32, _i32, _P(_sz)],
    "muon_update": [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _P(_f32), _i32, _f32, _f32, _f32,
                    _vp, _sz, _vp],
    "muon_update_noalloc": [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _P(_f32), _i32, _f32, _f32, _f32, _vp],
    "normuon_update": [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _P(_f32), _i32, _f32, _f32, _f32,
                       _f32, _f32, _vp, _sz, _vp],
    "gpt_op_gemm": [_i32, _i32, _i32, _i32, _vp, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _i32,
                    _i64, _i64, _f32, _f32, _vp],
    "gpt_op_attention_fwd": [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp],
    "gpt_op_attention_bwd": [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp,
                             _vp, _vp, _i64, _vp],
    "gpt_workspace_tensor": [_P(Shape), _i32, _i32, _P(_sz), _P(_sz)],
    "gpt_profile_enable": [ctypes.c_uint64],
    "gpt_profile_reset": [],
    "gpt_profile_read": [_i32, _P(ctypes.c_double), _P(_i32)],
    "gpt_probe_mfma": [_i32, _i32, _i32, _vp, _P(ctypes.c_double), _vp],
    "gpt_op_quantize_fp8": [_vp, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _i64, _vp, _i64, _vp, _vp],
    "gpt_op_gemm_fp8": [_i32, _i32, _i32, _vp, _i32, _i32, _i64, _vp, _i32, _i32, _i64, _vp, _i64, _vp, _vp, _f32, _vp],
}

EXPORTED = ["gpt_status_string", "gpt_last_error", "gpt_abi_version", "gpt_profile_num_categories",
            "gpt_profile_category_name", "gpt_fp8_partials"] + list(_SIGS)

for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name, None)
    if _f is None:
        continue
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.gpt_last_error.restype = ctypes.c_char_p
_lib.gpt_last_error.argtypes = []
_lib.gpt_status_string.restype = ctypes.c_char_p
_lib.gpt_status_string.argtypes = [ctypes.c_int]
_lib.gpt_abi_version.restype = ctypes.c_int32
_lib.gpt_profile_num_categories.restype = ctypes.c_int32
_lib.gpt_profile_category_name.restype = ctypes.c_char_p
_lib.gpt_profile_category_name.argtypes = [ctypes.c_int32]
_lib.gpt_fp8_partials.restype = ctypes.c_int32
_lib.gpt_fp8_partials.argtypes = [ctypes.c_int32, ctypes.c_int32]


def lib():
    return _lib


def _call(name, *args):
    fn = getattr(_lib, name)
    rc = fn(*args)
    if rc != 0:
        raise GptError(name, rc, _lib.gpt_last_error().decode())
    return rc


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def shape(depth, vocab, seq_len, batch, precision=PREC_BF16, n_kv_head=0, window=0, pattern="", features=""):
    """pattern: string of 'S' (windowed) / 'L' (full causal) layers, repeated
    over the depth (e.g. "SSSL"); empty = every layer full.  features: letters
    of the record-model features, "v" value embeddings, "s" smear, "r"
    per-layer residual scalars, "b" backout."""
    fbits = 0
    for ch in features:
        if ch not in FEATURE_BITS:
            raise ValueError("feature letters are v, s, r, b")
        fbits |= FEATURE_BITS[ch]
    bits = 0
    for i, ch in enumerate(pattern):
        if ch not in "SL":
            raise ValueError("pattern letters are S and L")
        if ch == "L":
            bits |= 1 << i
    return Shape(depth, vocab, seq_len, batch, precision, n_kv_head, window, len(pattern), bits, fbits)


def param_count(sh):
    n = _sz()
    _call("gpt_param_count", ctypes.byref(sh), ctypes.byref(n))
    return n.value


def param_layout(sh):
    n = _i32()
    cap = 2 + 7 * sh.depth + 6
    offs = (_sz * cap)()
    _call("gpt_param_layout", ctypes.byref(sh), offs, cap, ctypes.byref(n))
    return [offs[i] for i in range(n.value)]


def workspace_size(sh):
    n = _sz()
    _call("gpt_workspace_size", ctypes.byref(sh), ctypes.byref(n))
    return n.value


def workspace_tensor(sh, which, layer=0):
    off, nb = _sz(), _sz()
    _call("gpt_workspace_tensor", ctypes.byref(sh), which, layer, ctypes.byref(off), ctypes.byref(nb))
    return off.value, nb.value


def cast_bf16(src, dst, stream=None):
    assert src.dtype == torch.float32 and dst.dtype in (torch.bfloat16, torch.int16, torch.uint16)
    assert src.numel() == dst.numel()
    _call("gpt_cast_bf16", _ptr(src), _ptr(dst), src.numel(), _stream(stream))


def make_params(master, bf16, grad):
    return Params(_ptr(master), _ptr(bf16), _ptr(grad))


def step_fwd(sh, params, ids, loss, ws, row_lse=None, logits=None, stream=None):
    _call("gpt_step_fwd", ctypes.byref(sh), ctypes.byref(params), _ptr(ids), _ptr(loss),
          _ptr(row_lse), _ptr(logits), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))


def step_bwd(sh, params, ids, ws, accumulate=False, stream=None):
    _call("gpt_step_bwd", ctypes.byref(sh), ctypes.byref(params), _ptr(ids), int(accumulate),
          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))


def step_bwd_scaled(sh, params, ids, ws, loss_scale, accumulate=False, stream=None):
    _call("gpt_step_bwd_scaled", ctypes.byref(sh), ctypes.byref(params), _ptr(ids), int(accumulate),
          float(loss_scale), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))


def adamw_update(W, G, M, V, step, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, grad_scale=1.0,
                 W_bf16=None, stream=None):
    """W, G, M, V: fp32 tensors of the same number of elements."""
    n = W.numel()
    assert G.numel() == n and M.numel() == n and V.numel() == n
    _call("adamw_update", _ptr(W), _ptr(W_bf16), _ptr(G), _ptr(M), _ptr(V), n, int(step), lr, beta1, beta2, eps,
          weight_decay, grad_scale, _stream(stream))


def muon_workspace_size(count, rows, cols):
    n = _sz()
    _call("muon_workspace_size", count, rows, cols, ctypes.byref(n))
    return n.value


def muon_update(G, coeffs, ws, W=None, W_bf16=None, M=None, O_out=None, lr=0.02, momentum=0.95,
                weight_decay=0.0, stream=None):
    """G: fp32 [count, rows, cols] (or [rows, cols]); coeffs: list of (a, b, c)."""
    if G.dim() == 2:
        count, rows, cols = 1, G.shape[0], G.shape[1]
    else:
        count, rows, cols = G.shape
    flat = [float(x) for t in coeffs for x in t]
    carr = (_f32 * len(flat))(*flat)
    _call("muon_update", _ptr(W), _ptr(W_bf16), _ptr(G), _ptr(M), _ptr(O_out), count, rows, cols,
          carr, len(coeffs), lr, momentum, weight_decay, _ptr(ws), ws.numel() * ws.element_size(),
          _stream(stream))


def muon_update_noalloc(G, coeffs, W=None, W_bf16=None, M=None, O_out=None, lr=0.02, momentum=0.95,
                        weight_decay=0.0, stream=None):
    """muon_update with the library's own per-GPU scratch (no workspace, no
    allocation); raises GptError (code -3) when the shape needs more scratch."""
    if G.dim() == 2:
        count, rows, cols = 1, G.shape[0], G.shape[1]
    else:
        count, rows, cols = G.shape
    flat = [float(x) for t in coeffs for x in t]
    carr = (_f32 * len(flat))(*flat)
    _call("muon_update_noalloc", _ptr(W), _ptr(W_bf16), _ptr(G), _ptr(M), _ptr(O_out), count, rows, cols, carr,
          len(coeffs), lr, momentum, weight_decay, _stream(stream))


NOALLOC_SCRATCH_BYTES = 160 * 1024 * 1024


def normuon_update(G, coeffs, ws, V, W=None, W_bf16=None, M=None, O_out=None, lr=0.02, momentum=0.95,
                   weight_decay=0.0, beta2=0.95, eps=1e-8, per_row=True, stream=None):
    """Muon with the NorMuon per-neuron rescale; V: fp32 second moments, one
    per row (per_row) or column of each matrix, updated in place."""
    if G.dim() == 2:
        count, rows, cols = 1, G.shape[0], G.shape[1]
    else:
        count, rows, cols = G.shape
    flat = [float(x) for t in coeffs for x in t]
    carr = (_f32 * len(flat))(*flat)
    _call("normuon_update", _ptr(W), _ptr(W_bf16), _ptr(G), _ptr(M), _ptr(V), _ptr(O_out), count, rows, cols,
          int(bool(per_row)), carr, len(coeffs), lr, momentum, weight_decay, beta2, eps, _ptr(ws),
          ws.numel() * ws.element_size(), _stream(stream))


def gemm(A, B, C, M, N, K, a_layout=LAYOUT_K, b_layout=LAYOUT_K, lda=None, ldb=None, ldc=None,
         batch=1, stride_a=0, stride_b=0, stride_c=0, alpha=1.0, beta=0.0, stream=None):
    c_dtype = DTYPE_F32 if C.dtype == torch.float32 else DTYPE_BF16
    if lda is None:
        lda = K if a_layout == LAYOUT_K else M
    if ldb is None:
        ldb = K if b_layout == LAYOUT_K else N
    if ldc is None:
        ldc = N
    _call("gpt_op_gemm", M, N, K, batch, _ptr(A), a_layout, lda, stride_a, _ptr(B), b_layout, ldb,
          stride_b, _ptr(C), c_dtype, ldc, stride_c, alpha, beta, _stream(stream))


def attention_fwd(q, k, v, out, lse, batch, n_head, seq_len, ld_qkv, ld_out, n_kv_head=None, window=-1,
                  stream=None):
    _call("gpt_op_attention_fwd", batch, n_head, n_kv_head or n_head, seq_len, window, _ptr(q), _ptr(k), _ptr(v),
          ld_qkv, _ptr(out), ld_out, _ptr(lse), _stream(stream))


def attention_bwd(q, k, v, out, dout, lse, delta, dq_acc, dk, dv, batch, n_head, seq_len, ld_qkv,
                  ld_out, ld_dkv, n_kv_head=None, window=-1, stream=None):
    _call("gpt_op_attention_bwd", batch, n_head, n_kv_head or n_head, seq_len, window, _ptr(q), _ptr(k), _ptr(v),
          ld_qkv, _ptr(out), _ptr(dout), ld_out, _ptr(lse), _ptr(delta), _ptr(dq_acc), _ptr(dk), _ptr(dv),
          ld_dkv, _stream(stream))


def profile_categories():
    return [_lib.gpt_profile_category_name(i).decode() for i in range(_lib.gpt_profile_num_categories())]


def profile_enable(mask):
    _call("gpt_profile_enable", int(mask))


def profile_reset():
    _call("gpt_profile_reset")


def profile_read(cat):
    t, n = ctypes.c_double(), _i32()
    _call("gpt_profile_read", cat, ctypes.byref(t), ctypes.byref(n))
    return t.value, n.value


def probe_mfma(fp8, blocks, iters, out, stream=None):
    """Launch the matrix-core-only probe; returns the FLOPs of the launch."""
    f = ctypes.c_double()
    _call("gpt_probe_mfma", int(fp8), blocks, iters, _ptr(out), ctypes.byref(f), _stream(stream))
    return f.value


def fp8_partials(rows, cols):
    return int(_lib.gpt_fp8_partials(rows, cols))


def quantize_fp8(x, fmt, scale, partial, q=None, qt=None, rows=None, cols=None, ldx=None, ldq=None, ldqt=None,
                 stream=None):
    """Per-tensor fp8 codes of x [rows, cols] (bf16 or fp32): q [rows, cols]
    and / or qt [cols, rows] (uint8 tensors), scale (fp32 [1]) = fmax / amax."""
    if rows is None:
        rows, cols = x.shape
    x_dtype = DTYPE_F32 if x.dtype == torch.float32 else DTYPE_BF16
    _call("gpt_op_quantize_fp8", _ptr(x), x_dtype, ldx or cols, rows, cols, fmt, _ptr(scale), _ptr(q),
          ldq or cols, _ptr(qt), ldqt or rows, _ptr(partial), _stream(stream))


def gemm_fp8(A, fmt_a, B, fmt_b, C, M, N, K, scale_a, scale_b, lda=None, ldb=None, ldc=None, beta=0.0,
             a_layout=LAYOUT_K, b_layout=LAYOUT_K, stream=None):
    """C fp32 [M, N] = dec(A) dec(B)^T / (scale_a scale_b) (+ beta C); A and
    B uint8 codes, logically [M, K] and [N, K]: stored as such (LAYOUT_K) or
    transposed, [K, M] / [K, N] (LAYOUT_MN)."""
    lda = lda or (K if a_layout == LAYOUT_K else M)
    ldb = ldb or (K if b_layout == LAYOUT_K else N)
    _call("gpt_op_gemm_fp8", M, N, K, _ptr(A), fmt_a, a_layout, lda, _ptr(B), fmt_b, b_layout, ldb, _ptr(C),
          ldc or N, _ptr(scale_a), _ptr(scale_b), beta, _stream(stream))
