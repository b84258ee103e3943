"""Record-model features on the GPU (value embeddings, smear, per-layer
residual scalars, backout) against the oracle configured the same way: each
feature alone, all four together (also with grouped key/value heads and
window layers), the fp8 path, and gradient accumulation.

Bars: those of the whole-step parity test (loss relative error and row lse
rel L2 <= 1e-2; every gradient tensor, the value-embedding tables and gates
included, cosine >= 0.999 and rel L2 <= max(1e-2, 1.5 F) with F the
bf16-operand floor of that tensor); the fp8 run takes the fp8 bars of the fp8
parity test.

The scalar gradients (residual and x0 scalars, smear weight and scale,
backout scale) are single sums over all B*T*d stream elements whose terms
cancel: |sum t_i| is 1e-2 .. 2e-4 of sum |t_i| on these inputs.  A relative
bar on such a sum measures the cancellation, not the arithmetic, so each
element is held to the error bound of a sum whose terms each carry two bf16
roundings: |gpu - oracle| <= max(1e-2 |oracle|, 2^-8 sum |t_i|), with sum |t_i|
from the oracle (grad_abs); vectors also need cosine >= 0.999."""

import numpy as np
import pytest
import torch

from gpu_util import cosine, from_dev, rel_l2, say
from step_util import StepRun, oracle_run
from test_gpu_step import check_grads

pytestmark = pytest.mark.gpu

SCALARS = ("resid_lambda", "x0_lambda", "smear_w", "smear_lambda", "backout_lambda")


def check_scalars(got, ref, tau=2.0 ** -8, rel=1e-2, extra=None, cos_min=None):
    """Elementwise bar max(rel |ref|, tau * sum |terms|) (+ extra, an
    elementwise allowance) on the scalar gradients; cosine >= 0.999 (or
    cos_min[name]) for the vectors."""
    bad = []
    for name in SCALARS:
        g = np.asarray(got[name], dtype=np.float64)
        r = ref["grads"][name]
        bar = np.maximum(rel * np.abs(r), tau * ref["grad_abs"][name])
        if extra is not None:
            bar = np.maximum(bar, extra[name])
        err = np.abs(g - r)
        worst = float(np.max(err / np.maximum(bar, 1e-30)))
        say(f"  {name}: max |err| / bar {worst:.3f}  (gpu {g[:2]}, oracle {r[:2]})")
        if np.any(err > bar):
            bad.append(f"{name}: err {err} bar {bar}")
        cmin = 0.999 if cos_min is None else cos_min[name]
        if g.size > 1 and np.linalg.norm(r) > 0 and cosine(g, r) < cmin:
            bad.append(f"{name}: cos {cosine(g, r):.6f} (bar {cmin:.6f})")
    assert not bad, bad


def _without(d, names):
    return {k: v for k, v in d.items() if k not in names}

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
    floor = oracle_run(run, bf16_operands=True)
    got = run.grads()
    check_scalars(got, ref)
    check_grads(got, _without(ref["grads"], SCALARS), floor["grads"])


def test_features_fp8():
    from gpt_transformer_step_amd import binding as Bd
    say("features=vsrb fp8 depth=4 V=4096 T=256 B=2")
    run = StepRun(4, 4096, 256, 2, precision_flag=Bd.PREC_FP8, features="vsrb")
    run.fwd()
    run.bwd()
    torch.cuda.synchronize()
    loss = float(run.loss.item())
    ref = oracle_run(run, fp8=True, bf16_operands=True)
    f8x = oracle_run(run, fp8=True)
    fl = abs(ref["loss"] - f8x["loss"]) / abs(ref["loss"])
    say(f"  loss gpu {loss:.6f} fp8+bf16 oracle {ref['loss']:.6f} fp8 oracle {f8x['loss']:.6f}")
    assert abs(loss - ref["loss"]) / abs(ref["loss"]) <= max(1e-2, 1.5 * fl)
    grads = run.grads()
    # scalars: the conditioning bar, widened by the distance the fp8 oracle's
    # own bf16 rounding moves each of them; the cosine floor as for the other
    # fp8 gradients
    check_scalars(grads, ref, extra={n: 1.5 * np.abs(ref["grads"][n] - f8x["grads"][n]) for n in SCALARS},
                  cos_min={n: min(0.999, 1.0 - 1.5 * (1.0 - cosine(ref["grads"][n], f8x["grads"][n])))
                           for n in SCALARS})
    bad = []
    for name, r in _without(ref["grads"], SCALARS).items():
        g = np.asarray(grads[name], dtype=np.float64)
        assert np.all(np.isfinite(g)), name
        e, c = rel_l2(g, r), cosine(g, r)
        tol = max(1e-2, 1.5 * rel_l2(r, f8x["grads"][name]))
        cos_min = min(0.999, 1.0 - 1.5 * (1.0 - cosine(r, f8x["grads"][name])))
        if not (e <= tol and c >= cos_min):
            bad.append(f"{name}: rel_l2 {e:.2e} (bar {tol:.2e}) cos {c:.6f} (bar {cos_min:.6f})")
    say(f"  {len(ref['grads'])} gradients checked")
    assert not bad, bad


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
