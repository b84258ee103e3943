"""Write the full-size expected values used by tests/test_gpu_fullsize.py.

    python tests/golden/make_golden.py [d12 d20 d26 d20f8]

Calls only the oracle (and the seeded input generators).  For each workload
(depth 12 / 20 / 26 at T = 2048 with their batches, and d20f8 = depth 20,
T 2048, batch 4 in fp8) it runs one forward+backward of

  * the exact oracle (float32, nothing rounded: the function of the bf16
    weights), and
  * one member of the bf16 ensemble: the oracle's bf16 mode with
    jitter_seed=1 (d20f8: fp8 mode on top of it) -- one bf16 (fp8) computation
    of the step whose products were summed in another fp32 order,

and stores, for the exact run: the mean loss, the row log-sum-exp of 2048
sampled rows, and per gradient tensor its L2 norm and its block sketch
(sketch() below, float32); for the member: its loss, per tensor its norm, the
relative L2 distance of its full gradient from the exact one and the same
distance measured through the sketch.  The member's distances are the bf16
(fp8) spread that sets the comparison bar of each tensor.

The block sketch covers every element: the tensor is cut into 256 x 256 blocks
(zero padded) and each block B gives 64 numbers u_k^T B v_k, with u_k, v_k
random +-1 vectors drawn per tensor from PCG64 (seeded by the tensor's name).
For a difference E of two gradients, each number has mean 0 and variance
||E_block||^2, so the sketch's L2 norm estimates ||E|| to a relative standard
deviation of about sqrt(1 / (2 n)), n the number of projections (>= 576 here).
"""

import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from gpt_transformer_step_amd import inputs  # noqa: E402
from oracle import model as om  # noqa: E402
from oracle import precision  # noqa: E402

N_ROWS = 2048
SKETCH_PROJ = 64
SKETCH_BLOCK = 256
SAMPLE_SEED = 2718
WORKLOADS = {
    "d12": dict(inputs.WORKLOADS["d12"], fp8=False),
    "d20": dict(inputs.WORKLOADS["d20"], fp8=False),
    "d26": dict(inputs.WORKLOADS["d26"], fp8=False),
    # fp8 at the depth-20 shapes: 8192 tokens put the fc / proj products on
    # 256 x 256 tiles, the launches of the full step
    "d20f8": dict(depth=20, seq_len=2048, batch=4, fp8=True),
}


def sample_rows(n_rows_total):
    g = np.random.Generator(np.random.PCG64(SAMPLE_SEED))
    return np.sort(g.choice(n_rows_total, size=min(N_ROWS, n_rows_total), replace=False))


def _name_seed(name):
    return SAMPLE_SEED + sum(ord(ch) * (i + 1) for i, ch in enumerate(name))


def sign_vectors(name):
    """u, v: float64 [SKETCH_PROJ, SKETCH_BLOCK] of +-1, one pair per tensor."""
    g = np.random.Generator(np.random.PCG64(_name_seed(name)))
    s = g.integers(0, 2, size=(2, SKETCH_PROJ, SKETCH_BLOCK)) * 2.0 - 1.0
    return s[0], s[1]


def sketch(name, grad):
    """Block sketch of a gradient tensor (2-D [rows, cols]; 1-D as one row):
    float64 [SKETCH_PROJ * row_blocks * col_blocks]."""
    g = np.asarray(grad, dtype=np.float64)
    if g.ndim == 1:
        g = g[None, :]
    r, c = g.shape
    nb = SKETCH_BLOCK
    nbr, nbc = -(-r // nb), -(-c // nb)
    if (r, c) != (nbr * nb, nbc * nb):
        pad = np.zeros((nbr * nb, nbc * nb))
        pad[:r, :c] = g
        g = pad
    u, v = sign_vectors(name)
    t1 = np.tensordot(u, g.reshape(nbr, nb, nbc, nb), axes=([1], [1]))   # [proj, nbr, nbc, nb]
    return np.einsum("kabj,kj->kab", t1, v).ravel()


def sketch_noise(n_proj):
    """Relative standard deviation of a sketch-estimated distance."""
    return math.sqrt(1.0 / (2.0 * n_proj))


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def make(workload):
    wl = WORKLOADS[workload]
    depth, T, B, fp8 = wl["depth"], wl["seq_len"], wl["batch"], wl["fp8"]
    V = 32768
    dims = inputs.Dims.from_depth(depth, V)
    cfg = om.Config.from_depth(depth, V)
    master = inputs.master_weights(dims, inputs.SEED_W)
    P = inputs.unpack(dims, precision.round_bf16(master))
    ids = inputs.token_ids(B, T, V, inputs.SEED_IDS)
    out = {"ids_sha256": np.array(inputs.sha256(ids)), "weights_sha256": np.array(inputs.sha256(master)),
           "batch": np.array(B), "seq_len": np.array(T), "depth": np.array(depth), "fp8": np.array(fp8)}
    rows = sample_rows(B * T)
    out["rows"] = rows

    t0 = time.time()
    # GOLDEN_CACHE=<dir>: keep the exact run there and reuse it (the member
    # run of the largest workloads takes over an hour; an interrupted run then
    # restarts from the member)
    cache = os.environ.get("GOLDEN_CACHE")
    cpath = os.path.join(cache, f"exact_{workload}.npz") if cache else None
    if cpath and os.path.exists(cpath):
        C = np.load(cpath)
        ex = {"loss": float(C["loss"]), "lse": C["lse"],
              "grads": {k[2:]: C[k] for k in C.files if k.startswith("g.")}}
    else:
        ex = om.forward_backward(P, ids, cfg, dtype=np.float32, seq_chunk=1)
        if cpath:
            os.makedirs(cache, exist_ok=True)
            np.savez(cpath, loss=np.array(ex["loss"]), lse=ex["lse"],
                     **{"g." + k: v for k, v in ex["grads"].items()})
    out["exact.loss"] = np.array(ex["loss"])
    out["exact.lse"] = ex["lse"].reshape(-1)[rows].astype(np.float64)
    sk = {}
    for name, g in ex["grads"].items():
        sk[name] = sketch(name, g)
        out[f"exact.sketch.{name}"] = sk[name].astype(np.float32)
        out[f"exact.norm.{name}"] = np.array(np.linalg.norm(g.astype(np.float64)))
    print(f"{workload} exact: loss {ex['loss']:.6f} in {time.time() - t0:.0f} s", flush=True)
    exact_grads = ex["grads"]
    del ex

    t0 = time.time()
    mem = om.forward_backward(P, ids, cfg, dtype=np.float32, seq_chunk=None if fp8 else 1, fp8=fp8,
                              bf16_operands=True, jitter_seed=1)
    out["member.loss"] = np.array(mem["loss"])
    out["member.lse_rel"] = np.array(_rel(mem["lse"].reshape(-1)[rows], out["exact.lse"]))
    for name, g in mem["grads"].items():
        out[f"member.norm.{name}"] = np.array(np.linalg.norm(g.astype(np.float64)))
        out[f"member.dist.{name}"] = np.array(_rel(g, exact_grads[name]))
        out[f"member.sketch_dist.{name}"] = np.array(_rel(sketch(name, g), sk[name]))
    print(f"{workload} bf16{'+fp8' if fp8 else ''} member: loss {mem['loss']:.6f} in {time.time() - t0:.0f} s",
          flush=True)
    np.savez_compressed(os.path.join(HERE, f"fullsize_{workload}.npz"), **out)


if __name__ == "__main__":
    for w in (sys.argv[1:] or ["d12", "d20f8", "d20", "d26"]):
        make(w)
