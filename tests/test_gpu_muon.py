"""Muon parity: muon_update against the oracle's momentum + Newton-Schulz +
apply, on batches of same-shape matrices (square, tall, wide), and the
standalone Newton-Schulz on N(0,1) 1664x6656 and 1664x1664 matrices.

Bar (extension of the step's gradient bar): orthogonalised update rel L2
<= 1e-2 and cosine >= 0.999; updated weights rel L2 <= 1e-5 relative to W."""

import json
import os

import numpy as np
import pytest
import torch

from gpt_transformer_step_amd import inputs
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

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")
NS5 = [om.NS5_QUINTIC] * 5


def _tables():
    printed = [tuple(t) for t in json.load(open(GOLDEN))["polar_express_printed_triples"]]
    return {"ns5": NS5, "printed2": printed}


@pytest.fixture(scope="module")
def B():
    from gpt_transformer_step_amd import binding
    return binding


# (4, 1280, 1280) and (3, 1280, 2048) take the symmetric Gram / polynomial
# path (more 128x128 tiles than CUs); the latter also splits the Gram over K
@pytest.mark.parametrize("count,rows,cols", [(3, 256, 256), (2, 512, 128), (2, 128, 512), (1, 136, 200),
                                             (4, 1280, 1280), (3, 1280, 2048)])
@pytest.mark.parametrize("table", ["ns5", "printed2"])
def test_muon_update_parity(B, count, rows, cols, table):
    say(f"muon count={count} {rows}x{cols} table={table}")
    coeffs = _tables()[table]
    g = np.random.default_rng(rows * 3 + cols + count)
    W = g.standard_normal((count, rows, cols)).astype(np.float32) * 0.02
    G = g.standard_normal((count, rows, cols)).astype(np.float32) * 1e-3
    M = g.standard_normal((count, rows, cols)).astype(np.float32) * 1e-3
    dW, dG, dM = (torch.from_numpy(a).cuda() for a in (W, G, M))
    dWb = torch.empty((count, rows, cols), dtype=torch.bfloat16, device="cuda")
    dO = torch.empty((count, rows, cols), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.muon_workspace_size(count, rows, cols), dtype=torch.uint8, device="cuda")
    lr, mu, wd = 0.02, 0.95, 0.1
    B.muon_update(dG, coeffs, ws, W=dW, W_bf16=dWb, M=dM, O_out=dO, lr=lr, momentum=mu, weight_decay=wd)
    torch.cuda.synchronize()
    for i in range(count):
        Wn, Mn, O = om.muon_update(W[i], G[i], M[i], coeffs, lr, mu, wd)
        e, c = rel_l2(dO[i].cpu().numpy(), O), cosine(dO[i].cpu().numpy(), O)
        say(f"  [{i}] O rel_l2 {e:.3e} cos {c:.6f}")
        assert e <= 1e-2 and c >= 0.999
        assert rel_l2(dM[i].cpu().numpy(), Mn) < 1e-6
        assert np.abs(dW[i].cpu().numpy() - Wn).max() <= W_LINF * lr * np.abs(O).max() + 1e-6
        assert torch.equal(dWb[i], dW[i].to(torch.bfloat16))


@pytest.mark.parametrize("rows,cols", [(1664, 6656), (1664, 1664)])
def test_standalone_ns_full_size(B, rows, cols):
    say(f"standalone NS {rows}x{cols}")
    G = inputs.normal_matrix(rows, cols, inputs.SEED_NS)[0]
    dG = torch.from_numpy(G).cuda()
    dO = torch.empty_like(dG)
    ws = torch.empty(B.muon_workspace_size(1, rows, cols), dtype=torch.uint8, device="cuda")
    B.muon_update(dG, NS5, ws, O_out=dO)
    torch.cuda.synchronize()
    ref = om.newton_schulz(G, NS5)
    got = dO.cpu().numpy()
    e, c = rel_l2(got, ref), cosine(got, ref)
    say(f"  rel_l2 {e:.3e} cos {c:.6f}")
    assert e <= 1e-2 and c >= 0.999


# The groups one step updates, at the batch sizes the step uses: the S, F and
# P groups of the depth-20 model (4 x 20 [1280, 1280], 20 [5120, 1280], 20
# [1280, 5120]) and the depth-26 square group (4 x 26 [1664, 1664], ragged
# 256-row tiles).  These batches have more 256x256 tiles than the big-tile
# threshold, so the Gram and polynomial products run on 256x256 tiles with
# only the tiles on and above the diagonal computed and the bf16 copies
# mirrored -- the launches the benchmark times.  The whole batch runs in one
# call; three matrices (first, middle, last) are compared with the float64
# oracle.
BENCH_GROUPS = [(80, 1280, 1280), (20, 5120, 1280), (20, 1280, 5120), (104, 1664, 1664)]


def _group_inputs(count, rows, cols, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    W = g.standard_normal((count, rows, cols), dtype=np.float32) * np.float32(0.02)
    G = g.standard_normal((count, rows, cols), dtype=np.float32) * np.float32(1e-3)
    M = g.standard_normal((count, rows, cols), dtype=np.float32) * np.float32(1e-3)
    return W, G, M


@pytest.mark.parametrize("count,rows,cols", BENCH_GROUPS)
def test_muon_update_bench_groups(B, count, rows, cols):
    say(f"muon bench group count={count} {rows}x{cols}")
    W, G, M = _group_inputs(count, rows, cols, rows + cols + count)
    dW, dG, dM = (torch.from_numpy(a).cuda() for a in (W, G, M))
    dWb = torch.empty((count, rows, cols), dtype=torch.bfloat16, device="cuda")
    dO = torch.empty((count, rows, cols), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.muon_workspace_size(count, rows, cols), dtype=torch.uint8, device="cuda")
    lr, mu, wd = 0.02, 0.95, 0.1
    B.muon_update(dG, NS5, ws, W=dW, W_bf16=dWb, M=dM, O_out=dO, lr=lr, momentum=mu, weight_decay=wd)
    torch.cuda.synchronize()
    for i in (0, count // 2, count - 1):
        Wn, Mn, O = om.muon_update(W[i], G[i], M[i], NS5, lr, mu, wd)
        got = dO[i].cpu().numpy()
        e, c = rel_l2(got, O), cosine(got, O)
        say(f"  [{i}] O rel_l2 {e:.3e} cos {c:.6f}")
        assert e <= 1e-2 and c >= 0.999
        assert rel_l2(dM[i].cpu().numpy(), Mn) < 1e-6
        assert np.abs(dW[i].cpu().numpy() - Wn).max() <= W_LINF * lr * np.abs(O).max() + 1e-6
        assert torch.equal(dWb[i], dW[i].to(torch.bfloat16))


def test_muon_rejects_bad_args(B):
    G = torch.zeros((1, 64, 64), device="cuda")
    ws = torch.empty(B.muon_workspace_size(1, 64, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.GptError):
        B.muon_update(G, [], ws)
    with pytest.raises(B.GptError):
        B.muon_update(G, NS5, ws[:100])
    with pytest.raises(B.GptError):
        B.muon_update(G, [(float("nan"), 0.0, 0.0)], ws)
