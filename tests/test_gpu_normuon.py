"""NorMuon parity: normuon_update against the oracle's momentum +
Newton-Schulz + per-neuron rescale + apply, over two consecutive steps (so
the second-moment history matters), for square, tall and wide matrices and
both neuron axes.

Bars: the rescaled update O' rel L2 <= 1e-2 and cosine >= 0.999 (the Muon
bar); the second moments V rel L2 <= 1e-2 (they are mean squares of O, so
twice O's relative error); updated weights within W_LINF * lr * max|O'| of the
oracle's; the bf16 copy equal to the GPU's own fp32 weights rounded."""

import numpy as np
import pytest
import torch

from gpu_util import cosine, rel_l2, say
from oracle import muon as om

pytestmark = pytest.mark.gpu

# Elementwise bound on an updated weight, as a fraction of lr * max|O|.  The
# iterates are bf16 (dev.to "2. Optimizador Muon", NorMuon lines: the
# orthogonalised update is cast to float for its statistics and the scale is
# cast back to the update's dtype), so every element of O carries the
# roundings of its iterates: 2^-9 relative each, times |a| (1.875 for the
# textbook quintic) in the last update, accumulated over five updates --
# about 1 % of max|O| at worst (measured 1.1 %), against rel L2 2e-3 .. 4e-3.
W_LINF = 2e-2

NS5 = [om.NS5_QUINTIC] * 5


@pytest.fixture(scope="module")
def B():
    from gpt_transformer_step_amd import binding
    return binding


@pytest.mark.parametrize("count,rows,cols", [(3, 256, 256), (2, 512, 128), (2, 128, 512), (1, 136, 200),
                                             (2, 1280, 5120)])
@pytest.mark.parametrize("per_row", [True, False])
def test_normuon_update_parity(B, count, rows, cols, per_row):
    say(f"normuon count={count} {rows}x{cols} per_row={per_row}")
    g = np.random.default_rng(rows * 5 + cols + count + per_row)
    W = g.standard_normal((count, rows, cols)).astype(np.float32) * 0.02
    M = np.zeros((count, rows, cols), dtype=np.float32)
    nneur = rows if per_row else cols
    dW, dM = torch.from_numpy(W).cuda(), torch.from_numpy(M).cuda()
    dV = torch.zeros((count, nneur), dtype=torch.float32, device="cuda")
    dWb = torch.empty((count, rows, cols), dtype=torch.bfloat16, device="cuda")
    dO = torch.empty((count, rows, cols), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.muon_workspace_size(count, rows, cols), dtype=torch.uint8, device="cuda")
    lr, mu, wd, beta2, eps = 0.02, 0.95, 0.1, 0.9, 1e-8
    axis = 1 if per_row else 0
    rW = [W[i].astype(np.float64) for i in range(count)]
    rM = [np.zeros((rows, cols)) for _ in range(count)]
    rV = [np.zeros(nneur) for _ in range(count)]
    for step in range(2):
        # gradients with uneven neuron scales, so the rescale has work to do
        sc = np.exp(g.uniform(-2, 2, (count, rows, 1) if per_row else (count, 1, cols)))
        G = (g.standard_normal((count, rows, cols)) * sc * 1e-3).astype(np.float32)
        B.normuon_update(torch.from_numpy(G).cuda(), NS5, ws, dV, W=dW, W_bf16=dWb, M=dM, O_out=dO, lr=lr,
                         momentum=mu, weight_decay=wd, beta2=beta2, eps=eps, per_row=per_row)
        torch.cuda.synchronize()
        for i in range(count):
            rW[i], rM[i], O = om.normuon_update(rW[i], G[i], rM[i], rV[i], NS5, lr, mu, wd, beta2=beta2, eps_v=eps,
                                                axis=axis)
            got = dO[i].cpu().numpy()
            e, c = rel_l2(got, O), cosine(got, O)
            ev = rel_l2(dV[i].cpu().numpy(), rV[i])
            say(f"  step {step} [{i}] O' rel_l2 {e:.3e} cos {c:.6f}  V rel_l2 {ev:.3e}")
            assert e <= 1e-2 and c >= 0.999 and ev <= 1e-2
            assert rel_l2(dM[i].cpu().numpy(), rM[i]) < 1e-6
            assert np.abs(dW[i].cpu().numpy() - rW[i]).max() <= W_LINF * lr * np.abs(O).max() + 1e-6
            assert torch.equal(dWb[i], dW[i].to(torch.bfloat16))


def test_normuon_keeps_update_norm_on_gpu(B):
    """From V = 0 the rescale gives every neuron the RMS of the whole update
    (eps negligible) and keeps its Frobenius norm: checked on the GPU's own
    output against the plain Muon update of the same gradient."""
    count, rows, cols = 2, 384, 256
    g = np.random.default_rng(5)
    G = torch.from_numpy((g.standard_normal((count, rows, cols)) *
                          np.exp(g.uniform(-3, 3, (count, rows, 1)))).astype(np.float32)).cuda()
    ws = torch.empty(B.muon_workspace_size(count, rows, cols), dtype=torch.uint8, device="cuda")
    O_plain = torch.empty_like(G)
    O_nm = torch.empty_like(G)
    V = torch.zeros((count, rows), dtype=torch.float32, device="cuda")
    B.muon_update(G, NS5, ws, O_out=O_plain)
    B.normuon_update(G, NS5, ws, V, O_out=O_nm)
    torch.cuda.synchronize()
    for i in range(count):
        n0, n1 = O_plain[i].norm().item(), O_nm[i].norm().item()
        rms = O_nm[i].pow(2).mean(dim=1).sqrt().cpu().numpy()
        say(f"  [{i}] ||O|| {n0:.6f} ||O'|| {n1:.6f} neuron RMS spread {rms.max() / rms.min() - 1:.2e}")
        assert abs(n1 - n0) <= 1e-5 * n0
        assert np.allclose(rms, n0 / np.sqrt(rows * cols), rtol=1e-4)


# The depth-20 and depth-26 groups at the batch sizes the step uses (see the
# Muon test of the same name): the Newton-Schulz products take the 256x256
# symmetric tiles, and the per-neuron statistics run over full batches.  Two
# steps, so the second-moment history enters; three matrices compared.
BENCH_GROUPS = [(80, 1280, 1280), (20, 5120, 1280), (20, 1280, 5120), (104, 1664, 1664)]


@pytest.mark.parametrize("count,rows,cols", BENCH_GROUPS)
def test_normuon_update_bench_groups(B, count, rows, cols):
    per_row = True
    say(f"normuon bench group count={count} {rows}x{cols}")
    g = np.random.Generator(np.random.PCG64(rows * 7 + cols + count))
    W = g.standard_normal((count, rows, cols), dtype=np.float32) * np.float32(0.02)
    dW = torch.from_numpy(W).cuda()
    dM = torch.zeros((count, rows, cols), dtype=torch.float32, device="cuda")
    dV = torch.zeros((count, rows), dtype=torch.float32, device="cuda")
    dWb = torch.empty((count, rows, cols), dtype=torch.bfloat16, device="cuda")
    dO = torch.empty((count, rows, cols), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.muon_workspace_size(count, rows, cols), dtype=torch.uint8, device="cuda")
    lr, mu, wd, beta2, eps = 0.02, 0.95, 0.1, 0.95, 1e-8
    pick = (0, count // 2, count - 1)
    rW = {i: W[i].astype(np.float64) for i in pick}
    rM = {i: np.zeros((rows, cols)) for i in pick}
    rV = {i: np.zeros(rows) for i in pick}
    for step in range(2):
        sc = np.exp(g.uniform(-2, 2, (count, rows, 1))).astype(np.float32)
        G = g.standard_normal((count, rows, cols), dtype=np.float32) * sc * np.float32(1e-3)
        B.normuon_update(torch.from_numpy(G).cuda(), NS5, ws, dV, W=dW, W_bf16=dWb, M=dM, O_out=dO, lr=lr,
                         momentum=mu, weight_decay=wd, beta2=beta2, eps=eps, per_row=per_row)
        torch.cuda.synchronize()
        for i in pick:
            rW[i], rM[i], O = om.normuon_update(rW[i], G[i], rM[i], rV[i], NS5, lr, mu, wd, beta2=beta2, eps_v=eps,
                                                axis=1)
            got = dO[i].cpu().numpy()
            e, c = rel_l2(got, O), cosine(got, O)
            ev = rel_l2(dV[i].cpu().numpy(), rV[i])
            say(f"  step {step} [{i}] O' rel_l2 {e:.3e} cos {c:.6f}  V rel_l2 {ev:.3e}")
            assert e <= 1e-2 and c >= 0.999 and ev <= 1e-2
            assert np.abs(dW[i].cpu().numpy() - rW[i]).max() <= W_LINF * lr * np.abs(O).max() + 1e-6
            assert torch.equal(dWb[i], dW[i].to(torch.bfloat16))
