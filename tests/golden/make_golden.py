"""Write the full-size expected values used by tests/test_gpu_fullsize.py.

    python tests/golden/make_golden.py [d12 d20 d26]

Calls only the oracle (and the seeded input generators): for each workload it
runs one forward+backward of the exact oracle in float32 (one sequence at a
time) and of its bf16-operand mode, and stores
  * the mean loss, and the row log-sum-exp of 2048 sampled rows;
  * per gradient tensor: the full L2 norm and 1024 sampled elements (indices
    from a fixed PCG64 stream, recomputed by the test);
for both modes.  The bf16-operand values only set the tolerance floor of the
comparison (how far bf16 rounding of the activations moves each quantity).
"""

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
N_ELEMS = 1024
SAMPLE_SEED = 2718


def sample_rows(n_rows_total):
    g = np.random.Generator(np.random.PCG64(SAMPLE_SEED))
    return np.sort(g.choice(n_rows_total, size=min(N_ROWS, n_rows_total), replace=False))


def sample_elems(name, size):
    seed = SAMPLE_SEED + sum(ord(ch) * (i + 1) for i, ch in enumerate(name))
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(0, size, size=N_ELEMS)


def make(workload):
    wl = inputs.WORKLOADS[workload]
    depth, T, B = wl["depth"], wl["seq_len"], wl["batch"]
    V = 32768
    dims = inputs.Dims.from_depth(depth, V)
    cfg = om.Config.from_depth(depth, V)
    master = inputs.master_weights(dims, inputs.SEED_W)
    P = inputs.unpack(dims, precision.round_bf16(master))
    ids = inputs.token_ids(B, T, V, inputs.SEED_IDS)
    out = {"ids_sha256": np.array(inputs.sha256(ids)), "weights_sha256": np.array(inputs.sha256(master))}
    rows = sample_rows(B * T)
    out["rows"] = rows
    for mode, flag in (("exact", False), ("bf16ops", True)):
        t0 = time.time()
        r = om.forward_backward(P, ids, cfg, dtype=np.float32, seq_chunk=1, bf16_operands=flag)
        out[f"{mode}.loss"] = np.array(r["loss"])
        out[f"{mode}.lse"] = r["lse"].reshape(-1)[rows].astype(np.float64)
        for name, gten in r["grads"].items():
            flat = gten.reshape(-1)
            idx = sample_elems(name, flat.size)
            out[f"{mode}.norm.{name}"] = np.array(np.linalg.norm(flat.astype(np.float64)))
            out[f"{mode}.grad.{name}"] = flat[idx].astype(np.float64)
        print(f"{workload} {mode}: loss {r['loss']:.6f} in {time.time() - t0:.0f} s", flush=True)
        del r
    np.savez_compressed(os.path.join(HERE, f"fullsize_{workload}.npz"), **out)


if __name__ == "__main__":
    for w in (sys.argv[1:] or ["d12", "d20", "d26"]):
        make(w)
