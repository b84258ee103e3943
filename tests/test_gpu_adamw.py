"""AdamW (adamw_update) and gradient accumulation (gpt_step_bwd_scaled) on the
GPU against the oracle.

* AdamW: three steps with different gradients from a zero state; the update
  W_t - W_0 and the moments against the float64 oracle.  The GPU keeps W in
  fp32, so each step rounds W to 2^-24 of its size: the update's rel L2 bar is
  1e-6 + 4 * 2^-24 * ||W_0|| / ||update||; the moments (no such
  cancellation) within 1e-6.  The bf16 copy is bit-exact against
  round-to-nearest-even of the GPU's own fp32 weights.
* Accumulation: a batch of four sequences processed as two micro-batches of
  two (loss_scale = 1/(4 T), accumulate on the second) against the oracle's
  gradient of the mean loss over all four sequences, with the bars of the
  whole-step parity test.
"""

import numpy as np
import pytest
import torch

from gpu_util import cosine, rel_l2, say
from oracle import adamw as oadamw
from oracle import precision
from step_util import StepRun, check_rows, grad_rows, members, oracle_run
from gpt_transformer_step_amd import inputs

pytestmark = pytest.mark.gpu


def _B():
    from gpt_transformer_step_amd import binding
    return binding


@pytest.mark.parametrize("n", [4096, 1_000_004])
def test_adamw_matches_oracle(n):
    B = _B()
    say(f"adamw n={n}")
    g = np.random.default_rng(n)
    W0 = g.standard_normal(n).astype(np.float32)
    grads = [(g.standard_normal(n) * s).astype(np.float32) for s in (1.0, 0.05, 3.0)]
    hp = dict(lr=2e-3, beta1=0.8, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=0.5)
    W = torch.from_numpy(W0.copy()).cuda()
    Wb = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    M = torch.zeros(n, dtype=torch.float32, device="cuda")
    V = torch.zeros(n, dtype=torch.float32, device="cuda")
    rW, rM, rV = W0.astype(np.float64), np.zeros(n), np.zeros(n)
    for t, G in enumerate(grads, start=1):
        B.adamw_update(W, torch.from_numpy(G).cuda(), M, V, t, W_bf16=Wb, **hp)
        oadamw.adamw_update(rW, G, rM, rV, t, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                            hp["weight_decay"], hp["grad_scale"])
    torch.cuda.synchronize()
    w = W.cpu().numpy().astype(np.float64)
    e_upd = rel_l2(w - W0, rW - W0)
    e_m, e_v = rel_l2(M.cpu().numpy(), rM), rel_l2(V.cpu().numpy(), rV)
    bar = 1e-6 + 4 * 2.0 ** -24 * np.linalg.norm(W0) / np.linalg.norm(rW - W0)
    say(f"  update rel_l2 {e_upd:.2e} (bar {bar:.2e})  m {e_m:.2e}  v {e_v:.2e}")
    assert e_upd <= bar and e_m <= 1e-6 and e_v <= 1e-6
    bits = precision.bf16_bits(W.cpu().numpy())
    assert np.array_equal(Wb.view(torch.int16).cpu().numpy().view(np.uint16), bits)


def test_adamw_rejects_bad_args():
    B = _B()
    W = torch.zeros(8, dtype=torch.float32, device="cuda")
    with pytest.raises(B.GptError):
        B.adamw_update(W, W, W, W, 0, 1e-3)          # step is 1-based
    with pytest.raises(B.GptError):
        B.adamw_update(W, W, W, W, 1, 1e-3, beta1=1.0)


def test_gradient_accumulation_two_micro_batches():
    B = _B()
    depth, vocab, T, Bn, n_micro = 2, 4096, 128, 4, 2
    say(f"accumulation depth={depth} V={vocab} T={T} B={Bn} in {n_micro} micro-batches")
    mb = Bn // n_micro
    run = StepRun(depth, vocab, T, mb)
    ids_all = inputs.token_ids(Bn, T, vocab, inputs.SEED_IDS)
    for i in range(n_micro):
        run.ids = torch.from_numpy(np.ascontiguousarray(ids_all[i * mb:(i + 1) * mb])).cuda()
        run.fwd()
        B.step_bwd_scaled(run.shape, run.params, run.ids, run.ws, 1.0 / (Bn * T), accumulate=i > 0)
    torch.cuda.synchronize()
    grads = run.grads()
    run.ids_np = ids_all
    run.batch = Bn
    exact = oracle_run(run)
    check_rows(grad_rows(grads, exact["grads"], [m["grads"] for m in members(run)], 1e-2), "accumulated: ")
