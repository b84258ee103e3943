"""Record-model features on the GPU (value embeddings, smear, per-layer
residual scalars, backout) against the oracle configured the same way: each
feature alone, all four together (also with grouped key/value heads and
window layers), the fp8 path, and gradient accumulation.

Bars: those of the whole-step parity test (loss relative error and row lse
rel L2 <= 1e-2; every gradient tensor, the value-embedding tables and gates
included, against the exact oracle at max(1e-2, the bf16 ensemble's distance
(1 + kappa)) and cosine >= 0.999); the fp8 run takes the fp8 bars.

The scalar gradients (residual and x0 scalars, smear weight and scale,
backout scale) are single sums over all B*T*d stream elements whose terms
cancel.  Each element is held to max(1e-2 |exact|, 4 SCALAR_NOISE sum |terms|),
SCALAR_NOISE the measured rms error of a jittered bf16 run relative to the
sum of the terms' absolute values (the oracle's grad_abs); on the bf16
configurations below that bar is smaller than every scalar gradient except
near-zero components of the smear weight vector (covered by its cosine), so a
kernel that writes 0 fails.  fp8 adds its quantisation noise (rms up to
1.1e-3 of sum |terms|, measured the same way): the fp8 method itself cannot
resolve some of the scalars, and the fp8 test holds them to that noise."""

import numpy as np
import pytest
import torch

from gpu_util import cosine, from_dev, rel_l2, say
from step_util import StepRun, check_scalars, members, oracle_run
from test_gpu_step import check_grads

pytestmark = pytest.mark.gpu

SCALARS = ("resid_lambda", "x0_lambda", "smear_w", "smear_lambda", "backout_lambda")
# rms error of a jittered fp8 + bf16 run of the oracle on the scalar gradients,
# relative to sum |terms|: 1.4e-4 .. 1.1e-3 (depth 4, four seeds)
SCALAR_NOISE_FP8 = 1.2e-3


def _without(names, d):
    return [k for k in d if k not in names]


CONFIGS = [
    # depth, vocab, seq_len, batch, n_kv_head, window, pattern, features
    (4, 4096, 256, 2, 0, 0, "", "v"),
    (4, 4096, 256, 2, 0, 0, "", "s"),
    (4, 4096, 256, 2, 0, 0, "", "r"),
    (4, 4096, 256, 2, 0, 0, "", "b"),
    (4, 4096, 256, 2, 0, 0, "", "vsrb"),
    (6, 2048, 200, 2, 1, 50, "SL", "vsrb"),   # grouped heads, window layers, ragged T
    (2, 1000, 100, 3, 0, 0, "", "vsrb"),      # ragged vocabulary and token count
]


@pytest.mark.parametrize("depth,vocab,T,B,n_kv_head,window,pattern,features", CONFIGS)
def test_step_parity_features(depth, vocab, T, B, n_kv_head, window, pattern, features):
    say(f"features={features} depth={depth} V={vocab} T={T} B={B} n_kv_head={n_kv_head} window={window} "
        f"pattern={pattern}")
    run = StepRun(depth, vocab, T, B, n_kv_head=n_kv_head, window=window, pattern=pattern, features=features)
    run.fwd()
    run.bwd()
    torch.cuda.synchronize()
    ref = oracle_run(run)
    loss = float(run.loss.item())
    say(f"  loss gpu {loss:.6f} oracle {ref['loss']:.6f}")
    assert abs(loss - ref["loss"]) <= 1e-2 * abs(ref["loss"])
    e = rel_l2(from_dev(run.row_lse), ref["lse"].reshape(-1))
    say(f"  row lse rel_l2 {e:.3e}")
    assert e <= 1e-2
    got = run.grads()
    check_scalars(got, ref, SCALARS)
    check_grads(got, ref["grads"], members(run), names=_without(SCALARS, ref["grads"]))


def test_features_fp8():
    from gpt_transformer_step_amd import binding as Bd
    say("features=vsrb fp8 depth=4 V=4096 T=256 B=2")
    run = StepRun(4, 4096, 256, 2, precision_flag=Bd.PREC_FP8, features="vsrb")
    run.fwd()
    run.bwd()
    torch.cuda.synchronize()
    loss = float(run.loss.item())
    ref = oracle_run(run)
    say(f"  loss gpu {loss:.6f} exact oracle {ref['loss']:.6f}")
    assert abs(loss - ref["loss"]) / abs(ref["loss"]) <= 5e-2
    grads = run.grads()
    # the elementwise bar at the fp8 noise bounds every element; vectors of 4 to 24
    # noisy elements give no stable cosine, so none is asked for
    check_scalars(grads, ref, SCALARS, noise=SCALAR_NOISE_FP8, cos_min=-1.0)
    check_grads(grads, ref["grads"], members(run, fp8=True), base=5e-2, names=_without(SCALARS, ref["grads"]))


def test_features_accumulate_adds():
    run = StepRun(4, 1024, 64, 2, features="vsrb")
    run.fwd()
    run.bwd()
    torch.cuda.synchronize()
    g1 = run.grad.clone()
    run.bwd(accumulate=True)
    torch.cuda.synchronize()
    assert rel_l2(run.grad.cpu().numpy(), 2 * g1.cpu().numpy()) < 1e-5
    # the scalar block after two backward passes is twice the first
    off = run.B.param_layout(run.shape)
    sc = slice(off[-6], off[-1])
    assert np.allclose(run.grad[sc].cpu().numpy(), 2 * g1[sc].cpu().numpy(), rtol=1e-5, atol=1e-9)
