"""Whole-step parity: gpt_step_fwd / gpt_step_bwd against the oracle on the
same seeded token ids and bf16-valued weights.

Bars, against the exact float64 oracle (metrics in float64):
  * loss relative error <= 1e-2; row log-sum-exp and logits rel L2 <= 1e-2;
  * every gradient tensor: rel L2 <= max(1e-2, d_m (1 + kappa)) and cosine
    >= 0.999, d_m the distance of a jittered run of the oracle's bf16 mode
    (the precision passage's arithmetic with another fp32 summation order)
    from the exact gradient -- the spread no bf16 computation gets below (see
    step_util: on the q / k weights of deeper layers it is above 1e-2).
The target-logit pick is checked bit-exactly against the logits the same
kernel writes."""

import numpy as np
import pytest
import torch

from gpu_util import cosine, from_dev, rel_l2, say
from step_util import StepRun, check_rows, grad_rows, members, oracle_run

pytestmark = pytest.mark.gpu

CONFIGS = [
    # depth, vocab, seq_len, batch
    (2, 32768, 128, 2),   # the small configuration of the workload list
    (2, 1000, 100, 3),    # ragged: T and V not multiples of any tile
    (4, 4096, 256, 2),    # several attention tiles, two heads
]


def check_grads(got, exact, mems, base=1e-2, names=None, label=""):
    """Every gradient tensor against the exact oracle at the ensemble bar."""
    check_rows(grad_rows(got, exact, [m["grads"] for m in mems], base, names), label)


@pytest.mark.parametrize("depth,vocab,T,B", CONFIGS)
def test_step_parity(depth, vocab, T, B):
    say(f"step parity depth={depth} V={vocab} T={T} B={B}")
    run = StepRun(depth, vocab, T, B)
    want_logits = vocab * T * B <= 16 * 1024 * 1024
    logits = torch.empty((B * T, vocab), dtype=torch.float32, device="cuda") if want_logits else None
    run.fwd(logits=logits)
    run.bwd()
    torch.cuda.synchronize()
    ref = oracle_run(run, want_logits=want_logits)
    loss = float(run.loss.item())
    say(f"  loss gpu {loss:.6f} oracle {ref['loss']:.6f}")
    assert abs(loss - ref["loss"]) <= 1e-2 * abs(ref["loss"])
    e = rel_l2(from_dev(run.row_lse), ref["lse"].reshape(-1))
    say(f"  row lse rel_l2 {e:.3e}")
    assert e <= 1e-2
    if want_logits:
        lg = from_dev(logits)
        e = rel_l2(lg, ref["logits"])
        say(f"  logits rel_l2 {e:.3e}")
        assert e <= 1e-2
        # the target logit picked inside the fused kernel is exactly the
        # logit at the target column (same tile, same accumulation order)
        zt = run.ws_tensor(9).cpu().numpy()
        tgt = run.ids_np[:, 1:].reshape(-1)
        assert np.array_equal(zt, logits.cpu().numpy()[np.arange(len(tgt)), tgt])
    check_grads(run.grads(), ref["grads"], members(run))


GQA_WINDOW_CONFIGS = [
    # depth, vocab, seq_len, batch, n_kv_head, window, pattern
    (4, 4096, 256, 2, 1, 64, "SSSL"),    # two query heads share one key/value head
    (6, 2048, 200, 2, 3, 50, "SL"),      # plain heads, alternating window layers, ragged T
    (6, 1000, 130, 2, 1, 200, "S"),      # every layer windowed, window longer than T
]


@pytest.mark.parametrize("depth,vocab,T,B,n_kv_head,window,pattern", GQA_WINDOW_CONFIGS)
def test_step_parity_gqa_window(depth, vocab, T, B, n_kv_head, window, pattern):
    """Grouped key/value heads and sliding-window layers through the whole
    step, against the oracle configured the same way."""
    say(f"step parity depth={depth} V={vocab} T={T} B={B} n_kv_head={n_kv_head} window={window} "
        f"pattern={pattern}")
    run = StepRun(depth, vocab, T, B, n_kv_head=n_kv_head, window=window, pattern=pattern)
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
    check_grads(run.grads(), ref["grads"], members(run))


def test_bwd_accumulate_adds():
    run = StepRun(2, 1024, 64, 2)
    run.fwd()
    run.bwd()
    torch.cuda.synchronize()
    g1 = run.grad.clone()
    run.bwd(accumulate=True)
    torch.cuda.synchronize()
    assert rel_l2(run.grad.cpu().numpy(), 2 * g1.cpu().numpy()) < 1e-5


def test_repeat_is_deterministic_loss():
    run = StepRun(2, 2048, 128, 2)
    run.fwd()
    torch.cuda.synchronize()
    l1 = run.loss.item()
    run.fwd()
    torch.cuda.synchronize()
    assert run.loss.item() == l1


def test_embedding_gather_bit_exact():
    """x of a depth-2 model before any layer is wte[ids]; with all block
    weights zero the residual stream stays exactly the gathered rows."""
    run = StepRun(2, 512, 64, 2)
    off = run.B.param_layout(run.shape)
    # zero every block matrix: then attention and MLP add exactly 0
    with torch.no_grad():
        run.bf16[off[1]: off[-1]] = 0
    run.fwd()
    torch.cuda.synchronize()
    x = run.ws_tensor(0).cpu().numpy().reshape(run.batch * run.T, -1)
    wte = run.bf16[: off[1]].float().cpu().numpy().reshape(run.vocab, -1)
    inp = run.ids_np[:, :-1].reshape(-1)
    assert np.array_equal(x, wte[inp])


@pytest.mark.parametrize("features", ["", "vs"])
def test_out_of_range_ids_are_ignored(features):
    """An id outside [0, vocab) at position 0 of each sequence (an input,
    never a target) reads nothing and adds nothing: the step equals, bit for
    bit, the step with a valid unused id k there whose embedding (and
    value-embedding) rows are zero -- except the gradient of those rows,
    which is 0 with the out-of-range id."""
    depth, V, T, Bn = 2, 1024, 64, 2
    runs = {}
    for mode in ("oob", "zero_row"):
        run = StepRun(depth, V, T, Bn, features=features)
        ids = run.ids_np.copy()
        k = int(np.setdiff1d(np.arange(V), ids)[0])   # an id that appears nowhere
        ids[:, 0] = V + 7 if mode == "oob" else k
        run.ids = torch.from_numpy(ids).cuda()
        offs = run.B.param_layout(run.shape)
        d = 64 * depth
        with torch.no_grad():
            run.bf16[offs[0] + k * d: offs[0] + (k + 1) * d] = 0
            if "v" in features:
                for l in range(0, depth, 2):
                    ve = offs[2 + 6 * depth + l // 2]
                    run.bf16[ve + k * d: ve + (k + 1) * d] = 0
        run.fwd()
        run.bwd()
        torch.cuda.synchronize()
        runs[mode] = (float(run.loss.item()), run.grad.cpu().numpy(), offs, k)
    (la, ga, offs, k), (lb, gb, _, _) = runs["oob"], runs["zero_row"]
    say(f"  loss with id {V + 7}: {la:.6f}; with zero row {k}: {lb:.6f}")
    assert np.isfinite(la) and la == lb
    d = 64 * depth
    rows = [slice(offs[0] + k * d, offs[0] + (k + 1) * d)]
    if "v" in features:
        rows += [slice(offs[2 + 6 * depth + l // 2] + k * d, offs[2 + 6 * depth + l // 2] + (k + 1) * d)
                 for l in range(0, depth, 2)]
    for r in rows:
        assert np.all(ga[r] == 0)
        ga[r] = gb[r] = 0
    assert np.array_equal(ga, gb)
