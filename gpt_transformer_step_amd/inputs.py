"""Seeded synthetic inputs for the training step (no arithmetic of the method).

Both the tests of the HIP library and the oracle draw their inputs here, so
that both sides see identical arrays.  Nothing in this module computes any part
of the step; it only draws token ids and initial weights.

Stand-ins for the pages' data (dev.to "¿Cómo Entrenar Tu Propio ChatGPT por
$50?": ClimbMix tokens, vocabulary 32,768, sequence length 2048; per-GPU batch
16 or 32): token ids are uniform over the vocabulary (real text is Zipfian,
which changes only embedding-gradient collisions and the loss value, not the
work), weights are N(0, 1/fan_in) with fan_in the number of columns of the
stored [out, in] matrix, drawn from one PCG64 stream in packed order.  The
record-model scalars are drawn near their neutral values (residual scale
1 + 0.1 z, x0 scale 0.1 z, smear scale 0.5 + 0.1 z, backout scale
0.2 + 0.05 z) so that every term of the step is exercised.
"""

import hashlib
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Dims:
    """Tensor shapes of one model: n_layer blocks of width d_model; key/value
    projections of width d_kv = 128 * n_kv_head (d_model without grouping)."""
    n_layer: int
    d_model: int
    hidden: int
    vocab: int
    d_kv: int = 0
    features: str = ""     # record-model features: any of "v", "s", "r", "b"

    @staticmethod
    def from_depth(depth, vocab=32768, n_kv_head=0, features=""):
        d = 64 * depth
        return Dims(n_layer=depth, d_model=d, hidden=4 * d, vocab=vocab,
                    d_kv=128 * n_kv_head if n_kv_head else d, features=features)


SMEAR_CH = 24      # width of the smear gate's input
VE_GATE_CH = 32    # width of the value-embedding gate's input
SCALAR_PAD = 6     # unused tail of the scalar block (keeps the packed total a multiple of 4)


def packed_tensors(dims):
    """(name, shape) in packed parameter order: wte | per layer wq, wk, wv, wo |
    per layer wfc | per layer wproj | lm_head."""
    d, h, V, L = dims.d_model, dims.hidden, dims.vocab, dims.n_layer
    dkv = dims.d_kv or d
    out = [("wte", (V, d))]
    for i in range(L):
        out += [(f"wq.{i}", (d, d)), (f"wk.{i}", (dkv, d)), (f"wv.{i}", (dkv, d)), (f"wo.{i}", (d, d))]
    out += [(f"wfc.{i}", (h, d)) for i in range(L)]
    out += [(f"wproj.{i}", (d, h)) for i in range(L)]
    out.append(("lm_head", (V, d)))
    if dims.features:
        ve_layers = range(0, L, 2)
        out += [(f"ve.{i}", (V, dkv)) for i in ve_layers]
        out += [(f"ve_gate.{i}", (dkv // 128, VE_GATE_CH)) for i in ve_layers]
        out += [("resid_lambda", (L,)), ("x0_lambda", (L,)), ("smear_w", (SMEAR_CH,)), ("smear_lambda", (1,)),
                ("backout_lambda", (1,)), ("pad", (SCALAR_PAD,))]
    return out


# (offset, scale) of the scalar parameters: value = offset + scale * z
_SCALARS = {"resid_lambda": (1.0, 0.1), "x0_lambda": (0.0, 0.1), "smear_lambda": (0.5, 0.1),
            "backout_lambda": (0.2, 0.05), "pad": (0.0, 0.0)}


def n_params(dims):
    return sum(int(np.prod(s)) for _, s in packed_tensors(dims))


def token_ids(batch, seq_len, vocab, seed):
    """int32 [batch, seq_len + 1], uniform in [0, vocab)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(0, vocab, size=(batch, seq_len + 1), dtype=np.int32)


def master_weights(dims, seed, packed=None):
    """fp32 master weights as a flat packed array (float32 [n_params]).
    Each tensor is a float64 standard-normal block of the PCG64(seed) stream,
    scaled by 1/sqrt(fan_in), rounded to float32."""
    g = np.random.Generator(np.random.PCG64(seed))
    total = n_params(dims)
    out = np.empty(total, dtype=np.float32) if packed is None else packed
    off = 0
    for name, shape in packed_tensors(dims):
        n = int(np.prod(shape))
        if name in _SCALARS:
            base, sc = _SCALARS[name]
            out[off: off + n] = (base + sc * g.standard_normal(n)).astype(np.float32)
            off += n
            continue
        fan_in = shape[-1]
        # draw in slabs to bound the float64 temporary
        done = 0
        while done < n:
            k = min(n - done, 1 << 24)
            out[off + done: off + done + k] = (g.standard_normal(k) / np.sqrt(fan_in)).astype(np.float32)
            done += k
        off += n
    return out


def unpack(dims, flat):
    """Views of a packed flat array per tensor name."""
    out, off = {}, 0
    for name, shape in packed_tensors(dims):
        n = int(np.prod(shape))
        out[name] = flat[off: off + n].reshape(shape)
        off += n
    return out


def normal_matrix(rows, cols, seed, count=1):
    """float32 [count, rows, cols] of N(0, 1) from PCG64(seed)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.standard_normal((count, rows, cols), dtype=np.float32)


def sha256(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# Workloads: the configurations the step is measured and checked on.
WORKLOADS = {
    "d2": dict(depth=2, seq_len=128, batch=2),
    "d12": dict(depth=12, seq_len=2048, batch=16),
    "d20": dict(depth=20, seq_len=2048, batch=32),
    "d26": dict(depth=26, seq_len=2048, batch=16),
}
SEED_IDS = 1234
SEED_W = 5678
SEED_NS = 91011
