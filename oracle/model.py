"""Oracle forward and backward of one decoder-only GPT training step (numpy).

Test infrastructure only (see the package docstring).  Plain definitions, in
the order the pages describe the model, with hand-written backward formulas.

What the pages fix (dev.to "¿Cómo Entrenar Tu Propio ChatGPT por $50?",
section "Cómo Funciona nanochat" -> "1. Modelo GPT (nanochat/gpt.py)", and the
same list in apidog.com/pt "Modelo GPT"):
  * rotary position embeddings (RoPE), no learned positions;
  * QK normalisation of queries and keys;
  * token embedding and output matrix not tied;
  * ReLU squared in the MLP;
  * causal attention through ``flash_attn_func(q, k, v, causal=True, ...)``
    (section "5. Unificación Flash Attention");
  * vocabulary of 32,768 tokens (section "Lo que nanochat cubre").
Readings taken where the pages are silent:
  * pre-norm RMSNorm without gain, eps 1e-6 inside the square root, also
    used for the 128-wide QK normalisation; a final norm before the head;
  * RoPE base 10000, rotate-half pairing (i, i + hd/2), angle t * base^(-2i/hd),
    applied before the QK normalisation (the two commute: rotation keeps the
    per-head RMS);
  * full causal window, scale 1/sqrt(hd), multi-head (one KV head per head);
  * inputs ids[:, :T], targets ids[:, 1:], loss = mean over all B*T rows;
  * no biases, no logit soft-capping.

Attention variants (the same feature list: grouped-query attention with fewer
key/value heads, and sliding-window layers in a pattern such as "SSSL" that
alternates short and long context; the flash-attention call takes a
``window_size``):
  * n_kv_head key/value heads of width 128; query head h reads key/value head
    h // (n_head / n_kv_head), and a key/value head's gradient is the sum
    over its query heads;
  * window w (the left size of the flash-attention window): in an 'S' layer
    query i sees keys i - w .. i; 'L' layers are full causal; the pattern
    string repeats over the layers (layer i takes pattern[i % len]).

Record-model features (the same model section: value embeddings in the
ResFormer style, and the efficiency tricks -- per-layer residual scaling,
smear, backout; each a flag of Config).  The pages show one line or two of
each; the readings taken:
  * value embeddings (``value_embeds``): layers 0, 2, 4, ... ("alternating
    layers") own a table VE_i [V, n_kv_head * hd] gathered by the input
    token; gate = 3 sigmoid(h[:, :VE_GATE_CH] Wg_i^T) per key/value head, h
    being the attention's input (the normed stream) and Wg_i [n_kv_head,
    VE_GATE_CH] with VE_GATE_CH = 32 (the pages name the width, not its
    value); v <- v + gate * VE_i[ids] after the projection;
  * smear (``smear``): right after the embedding gather, token t >= 1 of a
    sequence adds gate_t times the previous token's embedding, gate_t =
    smear_lambda * sigmoid(e_t[:24] . smear_w) with e_t the token's own
    embedding (24 channels as printed); token 0 is unchanged;
  * per-layer residual scaling (``resid_lambdas``): layer i starts with
    x <- resid_lambda[i] x + x0_lambda[i] x0, x0 the stream after the
    embedding (and smear);
  * backout (``backout``): x_mid is the stream after layer L/2 - 1 (the
    middle); before the final norm x <- x - backout_lambda x_mid.
  The scalars and gates are parameters (the optimizer passage gives scalar
  parameters to AdamW); the extra tensors follow lm_head in packed order.

fp8 mode (``fp8=True``): the four block projections (qkv, out, fc, proj) use
per-tensor scaled fake quantisation as the precision passage describes
(apidog.com/pt "Gerenciamento de Precisão", apidog.com/de
"Präzisionsverwaltung": Float8Linear with tensorwise scaling): E4M3 for
activations and weights, E5M2 for output gradients, scale = fmax / amax of the
current tensor.  The fused q/k/v weight counts as one tensor.

Pinned by (tests/test_oracle_model.py): central finite differences in float64
of every parameter tensor on a tiny shape (also with grouped key/value heads
and windowed layers); brute-force double-loop causal and windowed attention; torch CPU autograd (float64) with torch's own RMS norm and
scaled-dot-product attention (with repeated key/value heads and an explicit
window mask for the variants) as an independent second implementation; the
closed form loss = ln V for a zero output matrix; softmax rows summing to 1;
RoPE identity at position 0, norm preservation and relative-position
invariance; RMSNorm output mean square = ms / (ms + eps).
"""

from dataclasses import dataclass

import numpy as np

from . import fp8 as _fp8
from . import precision as _precision


@dataclass(frozen=True)
class Config:
    n_layer: int
    d_model: int
    n_head: int
    head_dim: int
    hidden: int
    vocab: int
    eps: float = 1e-6
    rope_base: float = 10000.0
    n_kv_head: int = 0     # key/value heads (GQA); 0 = n_head
    window: int = 0        # 'S' layers: query i sees keys i - window .. i; 0 = every layer full
    pattern: str = "L"     # per-layer pattern, repeated over the layers ('S' short, 'L' long)
    value_embeds: bool = False
    smear: bool = False
    resid_lambdas: bool = False
    backout: bool = False

    @staticmethod
    def from_depth(depth, vocab=32768, n_kv_head=0, window=0, pattern="L", features=""):
        """Shapes from the single depth dial: width 64*depth, 128-wide heads,
        MLP 4x (dev.to page, "La Filosofía: Un Solo Selector").  features: any
        of "v" (value embeddings), "s" (smear), "r" (residual scaling), "b"
        (backout)."""
        d = 64 * depth
        return Config(n_layer=depth, d_model=d, n_head=d // 128, head_dim=128,
                      hidden=4 * d, vocab=vocab, n_kv_head=n_kv_head, window=window, pattern=pattern,
                      value_embeds="v" in features, smear="s" in features, resid_lambdas="r" in features,
                      backout="b" in features)

    @property
    def has_features(self):
        return self.value_embeds or self.smear or self.resid_lambdas or self.backout

    def ve_layers(self):
        """Layers with a value embedding (every other layer from the first)."""
        return list(range(0, self.n_layer, 2))

    @property
    def kv_heads(self):
        return self.n_kv_head or self.n_head

    def layer_window(self, i):
        """Left window of layer i (None: full causal)."""
        if self.window <= 0 or not self.pattern:
            return None
        return self.window if self.pattern[i % len(self.pattern)] == "S" else None


# ----------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------

SMEAR_CH = 24      # embedding channels feeding the smear gate (as printed)
BF16_JITTER = 2.0 ** -24   # relative perturbation before a bf16 rounding (fp32 unit roundoff)
VE_GATE_CH = 32    # channels of the attention input feeding the value-embedding gate


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def rms_norm(x, eps):
    """y = x / sqrt(mean(x^2) + eps) over the last axis; returns (y, r) with
    r = 1/sqrt(mean(x^2) + eps)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(ms + eps)
    return x * r, r


def rms_norm_bwd(dy, y, r):
    """Gradient of rms_norm: dx = r * (dy - y * mean(dy * y)), y the output."""
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def rope_tables(T, head_dim, base, dtype=np.float64):
    """cos/sin of angle t * base^(-2i/head_dim), t < T, i < head_dim/2
    (computed in float64)."""
    half = head_dim // 2
    inv_freq = base ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x, cos, sin):
    """Rotate pairs (i, i + hd/2) of the last axis by the position angle.
    x: [..., T, hd]; cos/sin: [T, hd/2]."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


def rope_bwd(dy, cos, sin):
    """Transpose of the rotation (the inverse rotation)."""
    half = dy.shape[-1] // 2
    d1, d2 = dy[..., :half], dy[..., half:]
    return np.concatenate([d1 * cos + d2 * sin, -d1 * sin + d2 * cos], axis=-1)


def attention_mask(T, window=None):
    """True where key j is hidden from query i: j > i, and with a window w
    also j < i - w (the query sees keys i - w .. i)."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    m = j > i
    if window is not None:
        m = m | (j < i - window)
    return m


def causal_attention(q, k, v, window=None, rnd=None):
    """softmax(q k^T / sqrt(hd) with masked keys removed) v (attention_mask).
    q, k, v: [..., T, hd].  Returns (y, lse) with lse the row log-sum-exp of
    the scaled, masked scores.  rnd (optional): the rounding applied to the
    probabilities as the operand of the product with v (bf16 mode)."""
    T, hd = q.shape[-2], q.shape[-1]
    s = (q @ np.swapaxes(k, -1, -2)) / np.sqrt(hd)
    mask = attention_mask(T, window)
    s = np.where(mask, -np.inf, s)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    den = np.sum(e, axis=-1, keepdims=True)
    p = e / den
    lse = (m + np.log(den))[..., 0]
    if rnd is not None:
        p = rnd(p)
    return p @ v, lse


def causal_attention_bwd(q, k, v, y, dy, lse, window=None, rnd=None):
    """Backward of causal_attention with P recomputed from lse:
    dV = P^T dY; dP = dY V^T; dS = P * (dP - rowsum(dY * Y)); dQ = dS K / sqrt(hd);
    dK = dS^T Q / sqrt(hd).  rnd (optional): the rounding applied to P and dS
    as operands of the products dV, dQ and dK (bf16 mode)."""
    T, hd = q.shape[-2], q.shape[-1]
    scale = 1.0 / np.sqrt(hd)
    s = (q @ np.swapaxes(k, -1, -2)) * scale
    mask = attention_mask(T, window)
    p = np.where(mask, 0.0, np.exp(s - lse[..., None]))
    dv = np.swapaxes(p if rnd is None else rnd(p), -1, -2) @ dy
    dp = dy @ np.swapaxes(v, -1, -2)
    dsum = np.sum(dy * y, axis=-1, keepdims=True)
    ds = p * (dp - dsum)
    if rnd is not None:
        ds = rnd(ds)
    dq = (ds @ k) * scale
    dk = (np.swapaxes(ds, -1, -2) @ q) * scale
    return dq, dk, dv


def cross_entropy(z, tgt):
    """Per-row loss lse(z) - z[tgt] with max-subtracted log-sum-exp.
    z: [R, V]; tgt: [R] int.  Returns (row_loss, lse)."""
    m = np.max(z, axis=-1, keepdims=True)
    lse = (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))[:, 0]
    picked = z[np.arange(z.shape[0]), tgt]
    return lse - picked, lse


def cross_entropy_bwd(z, tgt, lse, scale):
    """d(scale * sum row_loss)/dz = scale * (softmax(z) - onehot(tgt))."""
    dz = np.exp(z - lse[:, None])
    dz[np.arange(z.shape[0]), tgt] -= 1.0
    return dz * scale


# ----------------------------------------------------------------------------
# linear layers (bf16-valued weights; optional fp8 fake quantisation)
# ----------------------------------------------------------------------------

def _lin_fwd(x2, w, fp8):
    """y = x w^T for x [R, K], w [N, K]."""
    if fp8:
        x2 = _fp8.fake_quant(x2, "e4m3")
        w = _fp8.fake_quant(w, "e4m3")
    return x2 @ w.T


def _lin_bwd(x2, w, dy2, fp8):
    """dX = dY w, dW = dY^T x."""
    if fp8:
        dy2 = _fp8.fake_quant(dy2, "e5m2")
        w = _fp8.fake_quant(w, "e4m3")
        x2 = _fp8.fake_quant(x2, "e4m3")
    return dy2 @ w, dy2.T @ x2


# ----------------------------------------------------------------------------
# parameters
# ----------------------------------------------------------------------------

def param_names(cfg):
    """Parameter tensors in packed order: wte, per layer (wq, wk, wv, wo),
    per layer wfc, per layer wproj, lm_head; with any record-model feature
    then every value-embedding table, every value-embedding gate and the
    scalars (resid_lambda, x0_lambda, smear_w, smear_lambda, backout_lambda)."""
    names = ["wte"]
    for i in range(cfg.n_layer):
        names += [f"wq.{i}", f"wk.{i}", f"wv.{i}", f"wo.{i}"]
    names += [f"wfc.{i}" for i in range(cfg.n_layer)]
    names += [f"wproj.{i}" for i in range(cfg.n_layer)]
    names.append("lm_head")
    if cfg.has_features:
        names += [f"ve.{i}" for i in cfg.ve_layers()]
        names += [f"ve_gate.{i}" for i in cfg.ve_layers()]
        names += ["resid_lambda", "x0_lambda", "smear_w", "smear_lambda", "backout_lambda"]
    return names


def param_shapes(cfg):
    d, h, V, L = cfg.d_model, cfg.hidden, cfg.vocab, cfg.n_layer
    dkv = cfg.kv_heads * cfg.head_dim
    shapes = {}
    for n in param_names(cfg):
        base = n.split(".")[0]
        shapes[n] = {"wte": (V, d), "lm_head": (V, d), "wq": (d, d), "wk": (dkv, d),
                     "wv": (dkv, d), "wo": (d, d), "wfc": (h, d), "wproj": (d, h),
                     "ve": (V, dkv), "ve_gate": (cfg.kv_heads, VE_GATE_CH), "resid_lambda": (L,),
                     "x0_lambda": (L,), "smear_w": (SMEAR_CH,), "smear_lambda": (1,),
                     "backout_lambda": (1,)}[base]
    return shapes


# ----------------------------------------------------------------------------
# the step
# ----------------------------------------------------------------------------

def _forward_backward_chunk(P, ids, cfg, loss_scale, dtype, want_grads, want_logits, fp8, cos, sin, op, rnd):
    B, T1 = ids.shape
    T = T1 - 1
    d, H, hd = cfg.d_model, cfg.n_head, cfg.head_dim
    Hkv = cfg.kv_heads
    G = H // Hkv         # query heads per key/value head
    dkv = Hkv * hd
    R = B * T
    inp = ids[:, :T].reshape(-1)
    tgt = ids[:, 1:].reshape(-1)
    eps = cfg.eps

    L = cfg.n_layer
    ve_set = set(cfg.ve_layers()) if cfg.value_embeds else set()
    e = P["wte"][inp].astype(dtype)  # [R, d] token embeddings
    x = e
    if cfg.smear:
        # token t >= 1 adds gate_t * (embedding of token t-1) within its sequence
        e3 = e.reshape(B, T, d)
        prev = np.zeros_like(e3)
        prev[:, 1:] = e3[:, :-1]
        s_sig = sigmoid(e3[..., :SMEAR_CH] @ P["smear_w"])         # [B, T]
        s_gate = P["smear_lambda"][0] * s_sig
        s_gate[:, 0] = 0.0
        x = (e3 + s_gate[..., None] * prev).reshape(R, d)
    x0 = x
    x_mid = None
    caches = []
    for i in range(L):
        x_in = x
        if cfg.resid_lambdas:
            x = P["resid_lambda"][i] * x + P["x0_lambda"][i] * x0
        wqkv = np.concatenate([P[f"wq.{i}"], P[f"wk.{i}"], P[f"wv.{i}"]], axis=0)
        h1, r1 = rms_norm(x, eps)
        h1o = op(h1)
        qkv = _lin_fwd(h1o, wqkv, fp8)
        q_raw = qkv[:, :d].reshape(B, T, H, hd).transpose(0, 2, 1, 3)
        k_raw = qkv[:, d:d + dkv].reshape(B, T, Hkv, hd).transpose(0, 2, 1, 3)
        v_lin = qkv[:, d + dkv:]
        ve = v_gate = None
        if i in ve_set:
            # value embedding of the input token, gated per key/value head
            ve = P[f"ve.{i}"][inp].reshape(R, Hkv, hd)
            v_gate = 3.0 * sigmoid(h1o[:, :VE_GATE_CH] @ P[f"ve_gate.{i}"].T)   # [R, Hkv]
            v_lin = v_lin + (v_gate[:, :, None] * ve).reshape(R, dkv)
        v = op(v_lin.reshape(B, T, Hkv, hd).transpose(0, 2, 1, 3))
        qn, rq = rms_norm(rope(q_raw, cos, sin), eps)
        kn, rk = rms_norm(rope(k_raw, cos, sin), eps)
        qs, ks = op(qn), op(kn)
        # query head h reads key/value head h // G
        win = cfg.layer_window(i)
        y, lse_att = causal_attention(qs, np.repeat(ks, G, axis=1), np.repeat(v, G, axis=1), win, rnd=rnd)
        y2 = op(y.transpose(0, 2, 1, 3).reshape(R, d))
        x = x + _lin_fwd(y2, P[f"wo.{i}"], fp8)
        h2, r2 = rms_norm(x, eps)
        h2o = op(h2)
        u = _lin_fwd(h2o, P[f"wfc.{i}"], fp8)
        a = op(np.maximum(u, 0.0) ** 2)
        x = x + _lin_fwd(a, P[f"wproj.{i}"], fp8)
        caches.append((x_in, h1, h1o, r1, wqkv, qn, qs, rq, kn, ks, rk, v, ve, v_gate, y2, lse_att, h2, h2o,
                       r2, u, a))
        if cfg.backout and i == L // 2 - 1:
            x_mid = x

    if cfg.backout:
        x = x - P["backout_lambda"][0] * x_mid
    hf, rf = rms_norm(x, eps)
    hfo = op(hf)
    z = hfo @ P["lm_head"].T
    row_loss, lse = cross_entropy(z, tgt)
    out = {"row_loss": row_loss.reshape(B, T), "lse": lse.reshape(B, T),
           "loss_sum": float(np.sum(row_loss, dtype=np.float64))}
    if want_logits:
        out["logits"] = z
    if not want_grads:
        return out

    Gr = {}
    dz = op(cross_entropy_bwd(z, tgt, lse, loss_scale))
    del z
    Gr["lm_head"] = dz.T @ hfo
    g = rms_norm_bwd(op(dz @ P["lm_head"]), hfo, rf)
    del dz
    # the scalar gradients are sums over every stream element whose terms cancel
    # to a small fraction of their magnitudes; Gabs holds the sum of the
    # terms' absolute values (the scale that bounds a sum's rounding error)
    Gabs = {}
    if cfg.has_features:
        for n in ("resid_lambda", "x0_lambda", "smear_w", "smear_lambda", "backout_lambda"):
            Gr[n] = np.zeros(P[n].shape, dtype=dtype)
            Gabs[n] = np.zeros(P[n].shape, dtype=dtype)
    if cfg.backout:
        Gr["backout_lambda"][0] = -np.sum(g * x_mid)
        Gabs["backout_lambda"][0] = np.sum(np.abs(g * x_mid))
        g_mid = -P["backout_lambda"][0] * g
    g0 = np.zeros_like(g) if cfg.resid_lambdas else None   # gradient reaching x0 through the lambdas
    for i in reversed(range(L)):
        (x_in, h1, h1o, r1, wqkv, qn, qs, rq, kn, ks, rk, v, ve, v_gate, y2, lse_att, h2, h2o, r2, u,
         a) = caches[i]
        if cfg.backout and i == L // 2 - 1:
            g = g + g_mid
        # MLP
        gb = op(g)
        da, Gr[f"wproj.{i}"] = _lin_bwd(a, P[f"wproj.{i}"], gb, fp8)
        # d relu(u)^2 / du = 2 relu(u) = 2 sqrt(a), read from the stored activation
        du = op(da * 2.0 * np.sqrt(a))
        dh2, Gr[f"wfc.{i}"] = _lin_bwd(h2o, P[f"wfc.{i}"], du, fp8)
        g = g + rms_norm_bwd(op(dh2), h2o, r2)
        # attention
        gb = op(g)
        dy2, Gr[f"wo.{i}"] = _lin_bwd(y2, P[f"wo.{i}"], gb, fp8)
        dy = op(dy2).reshape(B, T, H, hd).transpose(0, 2, 1, 3)
        y = y2.reshape(B, T, H, hd).transpose(0, 2, 1, 3)
        dqn, dkf, dvf = causal_attention_bwd(qs, np.repeat(ks, G, axis=1), np.repeat(v, G, axis=1), y, dy,
                                             lse_att, cfg.layer_window(i), rnd=rnd)
        # a key/value head collects the gradients of its G query heads
        dkn = dkf.reshape(B, Hkv, G, T, hd).sum(axis=2)
        dv = dvf.reshape(B, Hkv, G, T, hd).sum(axis=2)
        dq = rope_bwd(rms_norm_bwd(dqn, qs, rq), cos, sin)
        dk = rope_bwd(rms_norm_bwd(dkn, ks, rk), cos, sin)
        dqkv = op(np.concatenate([t.transpose(0, 2, 1, 3).reshape(R, -1) for t in (dq, dk, dv)], axis=1))
        dh1, dwqkv = _lin_bwd(h1o, wqkv, dqkv, fp8)
        dh1 = op(dh1)
        Gr[f"wq.{i}"], Gr[f"wk.{i}"], Gr[f"wv.{i}"] = dwqkv[:d], dwqkv[d:d + dkv], dwqkv[d + dkv:]
        if ve is not None:
            dv3 = dqkv[:, d + dkv:].reshape(R, Hkv, hd)       # gradient of v after the value embedding
            dve = np.zeros(P[f"ve.{i}"].shape, dtype=dtype)
            np.add.at(dve, inp, (v_gate[:, :, None] * dv3).reshape(R, dkv))
            Gr[f"ve.{i}"] = dve
            # gate = 3 sigmoid(z): dgate/dz = gate (1 - gate / 3)
            dzg = np.sum(dv3 * ve, axis=-1) * v_gate * (1.0 - v_gate / 3.0)   # [R, Hkv]
            Gr[f"ve_gate.{i}"] = dzg.T @ h1o[:, :VE_GATE_CH]
            # the gate's share of dh1 joins the products' in the same bf16 tensor
            dh1 = dh1.copy()
            dh1[:, :VE_GATE_CH] = op(dh1[:, :VE_GATE_CH] + op(dzg @ P[f"ve_gate.{i}"]))
        g = g + rms_norm_bwd(dh1, h1o, r1)
        if cfg.resid_lambdas:
            # x = resid_lambda x_in + x0_lambda x0
            Gr["resid_lambda"][i] = np.sum(g * x_in)
            Gr["x0_lambda"][i] = np.sum(g * x0)
            Gabs["resid_lambda"][i] = np.sum(np.abs(g * x_in))
            Gabs["x0_lambda"][i] = np.sum(np.abs(g * x0))
            g0 += P["x0_lambda"][i] * g
            g = P["resid_lambda"][i] * g
        caches[i] = None
    if g0 is not None:
        g = g + g0
    if cfg.smear:
        # x_t = e_t + gate_t e_{t-1}, gate_t = lambda sigmoid(e_t[:24] . w)
        dX = g.reshape(B, T, d)
        de = dX.copy()
        de[:, :-1] += s_gate[:, 1:, None] * dX[:, 1:]
        dgate = np.sum(dX * prev, axis=-1)
        dgate[:, 0] = 0.0
        Gr["smear_lambda"][0] = np.sum(dgate * s_sig)
        Gabs["smear_lambda"][0] = np.sum(np.abs(dX * prev) * s_sig[..., None])
        dzs = dgate * P["smear_lambda"][0] * s_sig * (1.0 - s_sig)
        Gr["smear_w"] = np.einsum("bt,btc->c", dzs, e3[..., :SMEAR_CH])
        # dz_t itself is a sum over the channels of dX_t e_{t-1}
        dzs_abs = np.sum(np.abs(dX * prev), axis=-1) * abs(P["smear_lambda"][0]) * s_sig * (1.0 - s_sig)
        Gabs["smear_w"] = np.einsum("bt,btc->c", dzs_abs, np.abs(e3[..., :SMEAR_CH]))
        de[..., :SMEAR_CH] += dzs[..., None] * P["smear_w"]
        g = de.reshape(R, d)
    dwte = np.zeros(P["wte"].shape, dtype=dtype)
    np.add.at(dwte, inp, g)
    Gr["wte"] = dwte
    for i in (range(L) if cfg.has_features else ()):
        if f"ve.{i}" in P and f"ve.{i}" not in Gr:
            Gr[f"ve.{i}"] = np.zeros(P[f"ve.{i}"].shape, dtype=dtype)
            Gr[f"ve_gate.{i}"] = np.zeros(P[f"ve_gate.{i}"].shape, dtype=dtype)
    out["grads"] = Gr
    out["grad_abs"] = Gabs
    return out


def forward_backward(P, ids, cfg, dtype=np.float64, want_grads=True, want_logits=False,
                     fp8=False, seq_chunk=None, bf16_operands=False, jitter_seed=None):
    """One training step's forward and backward.

    P: dict name -> array (the bf16-rounded weight values, see precision.py);
    ids: int array [B, T+1].  Returns dict with ``loss`` (mean over B*T rows),
    ``row_loss`` and ``lse`` [B, T], optional ``logits`` [B*T, V] and ``grads``
    (dict name -> gradient of ``loss``).

    seq_chunk: process that many sequences at a time (the sequences of a batch
    are independent up to the loss mean); not allowed with fp8, whose
    per-tensor scales span the whole batch.

    bf16_operands: the precision passage's compute dtype (dev.to "3. Gestión
    de Precisión": the weight is cast to the activation's dtype for every
    matrix product, bf16 on bf16-capable GPUs; the flash-attention call takes
    bf16 q, k, v).  Reading taken: every operand of every matrix product holds
    bf16 values, and an activation is kept once, in bf16, for the backward.
    Rounded (nearest even), in the forward: the normed block inputs h1, h2
    and the head input; q and k after rotary + QK norm; v; the attention
    probabilities P as the operand of P v; the attention output; the ReLU^2
    output a.  In the backward: dlogits; the residual gradient entering the
    output projections' products; the MLP hidden gradient du; the attention
    output gradient dO; P and dS as operands of dV = P^T dO, dQ = dS K and
    dK = dS^T Q; the q/k/v gradient; the data gradient entering each RMS-norm
    backward (the head's, the fc product's, the q/k/v product's -- with value
    embeddings the gate's share is rounded and added to the latter in bf16).
    The ReLU^2 derivative 2 relu(u) is read
    from the stored activation as 2 sqrt(a), and each RMS-norm backward reads
    its stored (rounded) output.  Products accumulate in `dtype`; norm
    statistics, rotary, softmax and the residual stream stay in `dtype`.
    With False (default) nothing is rounded and the result is the exact
    function of the bf16 weights (2 sqrt(relu(u)^2) = 2 relu(u) exactly).

    jitter_seed (bf16 mode only): every value is multiplied by
    (1 + 2^-24 xi), xi ~ N(0, 1) from PCG64(jitter_seed), right before it is
    rounded to bf16.  2^-24 is the fp32 unit roundoff: each seed gives one
    more bf16 computation of the step whose products were summed in another
    fp32 order.  A chain of bf16 roundings is chaotic at the level of its own
    rounding noise (a relative change far below one bf16 ulp flips a few
    roundings, whose changes flip more), so a set of seeds measures how far
    any bf16 computation of the step lands from the exact result -- the
    spread a correct bf16 implementation cannot get below.

    ``grad_abs`` (with the record-model features): for each scalar parameter's
    gradient, a sum over every stream element, the sum of its terms' absolute
    values.  Those sums cancel to 1e-2 .. 1e-4 of that scale, so it, not the
    gradient's own size, bounds the gradient's rounding error."""
    ids = np.asarray(ids)
    B, T1 = ids.shape
    T = T1 - 1
    P = {k: np.asarray(v, dtype=dtype) for k, v in P.items()}
    cos, sin = rope_tables(T, cfg.head_dim, cfg.rope_base, dtype)
    if jitter_seed is not None and not bf16_operands:
        raise ValueError("jitter_seed perturbs the bf16 roundings; it needs bf16_operands=True")
    jit = np.random.Generator(np.random.PCG64(jitter_seed)) if jitter_seed is not None else None
    if bf16_operands:
        def op(t):
            if jit is not None:
                t = t * (1.0 + BF16_JITTER * jit.standard_normal(np.shape(t)))
            return _precision.round_bf16(t).astype(dtype)
        rnd = op
    else:
        def op(t):
            return t
        rnd = None
    loss_scale = 1.0 / (B * T)
    if seq_chunk is None or seq_chunk >= B:
        chunks = [(0, B)]
    else:
        if fp8:
            raise ValueError("fp8 per-tensor scales need the whole batch at once")
        chunks = [(s, min(B, s + seq_chunk)) for s in range(0, B, seq_chunk)]
    total, grads, gabs, row_loss, lse, logits = 0.0, None, None, [], [], []
    for s, e in chunks:
        o = _forward_backward_chunk(P, ids[s:e], cfg, loss_scale, dtype, want_grads,
                                    want_logits, fp8, cos, sin, op, rnd)
        total += o["loss_sum"]
        row_loss.append(o["row_loss"])
        lse.append(o["lse"])
        if want_logits:
            logits.append(o["logits"])
        if want_grads:
            if grads is None:
                grads, gabs = o["grads"], o["grad_abs"]
            else:
                for k in grads:
                    grads[k] += o["grads"][k]
                for k in gabs:
                    gabs[k] += o["grad_abs"][k]
    out = {"loss": total / (B * T), "row_loss": np.concatenate(row_loss),
           "lse": np.concatenate(lse)}
    if want_logits:
        out["logits"] = np.concatenate(logits)
    if want_grads:
        out["grads"] = grads
        out["grad_abs"] = gabs
    return out

