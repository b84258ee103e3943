"""Whole-step parity at the full workload sizes (depth 12, 20, 26; T = 2048;
B = 16 / 32 / 16; V = 32768), in the launch configuration bench.py times.

The expected values come from tests/golden/make_golden.py, which runs only
the oracle (float32, one sequence at a time) on the same seeded inputs and
stores: the loss, the row log-sum-exp of sampled rows, and for every gradient
tensor its L2 norm and sampled elements, for the exact oracle and for its
bf16-operand mode (which measures the bf16 noise floor of each quantity).

Bars: loss relative error <= 1e-2; sampled row lse rel L2 <= 1e-2; per
gradient tensor, on the sampled elements, cosine >= 0.999 and rel L2 <=
max(1e-2, 1.5 F) with F the bf16 floor on the same elements; and the full
gradient norm within the same relative bar."""

import os
import sys

import numpy as np
import pytest
import torch

from gpu_util import cosine, rel_l2, say
from step_util import StepRun

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_golden  # noqa: E402

from gpt_transformer_step_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", ["d12", "d20", "d26"])
def test_fullsize_step(wl):
    path = os.path.join(HERE, "golden", f"fullsize_{wl}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    G = np.load(path)
    cfg = inputs.WORKLOADS[wl]
    say(f"full-size step parity {wl}: depth={cfg['depth']} T={cfg['seq_len']} B={cfg['batch']}")
    run = StepRun(cfg["depth"], 32768, cfg["seq_len"], cfg["batch"])
    assert str(G["ids_sha256"]) == inputs.sha256(run.ids_np)
    assert str(G["weights_sha256"]) == inputs.sha256(run.master_np)
    run.fwd()
    run.bwd()
    torch.cuda.synchronize()

    loss = float(run.loss.item())
    ref_loss = float(G["exact.loss"])
    say(f"  loss gpu {loss:.6f} oracle {ref_loss:.6f} (bf16-operand oracle {float(G['bf16ops.loss']):.6f})")
    assert abs(loss - ref_loss) <= 1e-2 * abs(ref_loss)

    rows = G["rows"]
    lse = run.row_lse.cpu().numpy().astype(np.float64)[rows]
    e_lse = rel_l2(lse, G["exact.lse"])
    say(f"  row lse rel_l2 {e_lse:.3e}")
    assert e_lse <= 1e-2

    offs = run.B.param_layout(run.shape)
    names = [n for n, _ in inputs.packed_tensors(run.dims)]
    sizes = [int(np.prod(s)) for _, s in inputs.packed_tensors(run.dims)]
    flat = run.grad
    bad, worst = [], (0.0, "")
    for name, off, size in zip(names, offs, sizes):
        idx = make_golden.sample_elems(name, size)
        got = flat[off: off + size][torch.from_numpy(idx).to(flat.device)].cpu().numpy().astype(np.float64)
        ref = G[f"exact.grad.{name}"]
        floor = rel_l2(G[f"bf16ops.grad.{name}"], ref)
        tol = max(1e-2, 1.5 * floor)
        e, c = rel_l2(got, ref), cosine(got, ref)
        nrm = float(torch.linalg.vector_norm(flat[off: off + size].double()).item())
        ref_n = float(G[f"exact.norm.{name}"])
        floor_n = abs(float(G[f"bf16ops.norm.{name}"]) - ref_n) / ref_n
        e_n = abs(nrm - ref_n) / ref_n
        tol_n = max(1e-2, 1.5 * floor_n)
        if e / tol > worst[0]:
            worst = (e / tol, f"{name}: rel_l2 {e:.3e} floor {floor:.3e} cos {c:.6f} norm err {e_n:.2e}")
        if not (e <= tol and c >= 0.999 and e_n <= tol_n):
            bad.append(f"{name}: rel_l2 {e:.3e} (floor {floor:.3e}) cos {c:.6f} norm err {e_n:.2e} "
                       f"(floor {floor_n:.2e})")
    say(f"  worst gradient vs its bar: {worst[1]}")
    assert not bad, bad
