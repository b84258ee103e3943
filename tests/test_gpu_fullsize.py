"""Whole-step parity at the full workload sizes (depth 12, 20, 26 at T = 2048
with batches 16 / 32 / 16, V = 32768, bf16; depth 20 at T = 2048, B = 4 in
fp8), in the launch configuration bench.py times.

The expected values come from tests/golden/make_golden.py, which runs only the
oracle on the same seeded inputs: the exact step (float32) and one jittered
run of its bf16 mode (fp8 mode on top for the fp8 workload).  They hold the
loss, the row log-sum-exp of 2048 sampled rows, and for every gradient tensor
its norm and its block sketch -- 64 random +-1 projections u^T B v of every
256 x 256 block, so every element counts -- plus the member's distance from
the exact gradient measured through the same sketch.

Bars: loss relative error and sampled row lse rel L2 <= 1e-2 (fp8: 5e-2); per
gradient tensor, the sketch-measured rel L2 from the exact gradient <=
max(1e-2 (fp8: 5e-2), d_m (1 + kappa)) and the sketch cosine >= 0.999 (fp8:
what d_m (1 + kappa) allows), d_m the member's sketch distance and kappa =
4 sqrt(RHO^2 + 1/n) (the member spread and the sampling noise of two sketch
estimates over n projections); the gradient norm within the same relative
bar."""

import math
import os
import sys

import numpy as np
import pytest
import torch

from gpu_util import cosine, rel_l2, say
from step_util import RHO, StepRun

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_golden  # noqa: E402

from gpt_transformer_step_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", ["d12", "d20", "d26", "d20f8"])
def test_fullsize_step(wl):
    from gpt_transformer_step_amd import binding as Bd
    path = os.path.join(HERE, "golden", f"fullsize_{wl}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    G = np.load(path)
    if "exact.sketch.wte" not in G.files:
        pytest.skip(f"{path} predates the sketch format; rerun tests/golden/make_golden.py {wl}")
    cfg = make_golden.WORKLOADS[wl]
    fp8 = cfg["fp8"]
    base = 5e-2 if fp8 else 1e-2
    say(f"full-size step parity {wl}: depth={cfg['depth']} T={cfg['seq_len']} B={cfg['batch']} fp8={fp8}")
    run = StepRun(cfg["depth"], 32768, cfg["seq_len"], cfg["batch"], precision_flag=Bd.PREC_FP8 if fp8 else 0)
    assert str(G["ids_sha256"]) == inputs.sha256(run.ids_np)
    assert str(G["weights_sha256"]) == inputs.sha256(run.master_np)
    run.fwd()
    run.bwd()
    torch.cuda.synchronize()

    loss = float(run.loss.item())
    ref_loss = float(G["exact.loss"])
    say(f"  loss gpu {loss:.6f} oracle {ref_loss:.6f} (member {float(G['member.loss']):.6f})")
    assert abs(loss - ref_loss) <= base * abs(ref_loss)

    rows = G["rows"]
    lse = run.row_lse.cpu().numpy().astype(np.float64)[rows]
    e_lse = rel_l2(lse, G["exact.lse"])
    say(f"  row lse rel_l2 {e_lse:.3e} (member {float(G['member.lse_rel']):.3e})")
    assert e_lse <= base

    offs = run.B.param_layout(run.shape)
    tensors = inputs.packed_tensors(run.dims)
    flat = run.grad
    bad, worst, n_flat = [], (0.0, ""), 0
    for (name, shape), off in zip(tensors, offs):
        size = int(np.prod(shape))
        g = flat[off: off + size].cpu().numpy().reshape(shape)
        s_ex = G[f"exact.sketch.{name}"].astype(np.float64)
        s_gpu = make_golden.sketch(name, g)
        d, c = rel_l2(s_gpu, s_ex), cosine(s_gpu, s_ex)
        dm = float(G[f"member.sketch_dist.{name}"])
        kappa = 4.0 * math.sqrt(RHO ** 2 + 1.0 / s_ex.size)
        bar = max(base, dm * (1.0 + kappa))
        n_flat += bar == base
        cbar = 0.999 if not fp8 else min(0.999, 1.0 - 0.5 * (dm * (1.0 + kappa)) ** 2)
        nrm = float(np.linalg.norm(g.astype(np.float64)))
        ref_n = float(G[f"exact.norm.{name}"])
        e_n = abs(nrm - ref_n) / ref_n
        mem_n = abs(float(G[f"member.norm.{name}"]) - ref_n) / ref_n
        bar_n = max(base, mem_n * (1.0 + kappa))
        if d / bar > worst[0]:
            worst = (d / bar, f"{name}: rel_l2 {d:.3e} (member {dm:.3e}, bar {bar:.3e}) cos {c:.6f} "
                              f"norm err {e_n:.2e} (member {mem_n:.2e})")
        if not (d <= bar and c >= cbar and e_n <= bar_n):
            bad.append(f"{name}: rel_l2 {d:.3e} (member {dm:.3e}, bar {bar:.3e}) cos {c:.6f} (bar {cbar:.6f}) "
                       f"norm err {e_n:.2e} (bar {bar_n:.2e})")
    say(f"  worst gradient vs its bar: {worst[1]}; {n_flat}/{len(tensors)} tensors at the flat {base:g} bar")
    assert not bad, bad
