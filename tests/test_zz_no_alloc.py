"""muon_update_noalloc: the Muon update through the library's own per-GPU
scratch array (no workspace argument, no allocation) gives exactly what
muon_update gives with a caller workspace -- the same kernels on the same
inputs, so the outputs (orthogonalised update, momentum, fp32 and bf16
weights) are compared bit for bit -- on two calls in a row, the second with a
smaller input (the array keeps the first call's contents), and a shape that
needs more scratch than the array holds is rejected with GPT_ERR_WORKSPACE."""

import numpy as np
import pytest
import torch

from gpu_util import say
from oracle import muon as om

pytestmark = pytest.mark.gpu

NS5 = [om.NS5_QUINTIC] * 5


@pytest.fixture(scope="module")
def B():
    from gpt_transformer_step_amd import binding
    return binding


def _run(B, count, rows, cols, seed, noalloc):
    g = np.random.Generator(np.random.PCG64(seed))
    W = torch.from_numpy(g.standard_normal((count, rows, cols), dtype=np.float32) * np.float32(0.02)).cuda()
    G = torch.from_numpy(g.standard_normal((count, rows, cols), dtype=np.float32) * np.float32(1e-3)).cuda()
    M = torch.from_numpy(g.standard_normal((count, rows, cols), dtype=np.float32) * np.float32(1e-3)).cuda()
    Wb = torch.empty((count, rows, cols), dtype=torch.bfloat16, device="cuda")
    O = torch.empty((count, rows, cols), dtype=torch.float32, device="cuda")
    kw = dict(W=W, W_bf16=Wb, M=M, O_out=O, lr=0.02, momentum=0.95, weight_decay=0.1)
    if noalloc:
        B.muon_update_noalloc(G, NS5, **kw)
    else:
        ws = torch.empty(B.muon_workspace_size(count, rows, cols), dtype=torch.uint8, device="cuda")
        B.muon_update(G, NS5, ws, **kw)
    torch.cuda.synchronize()
    return O, M, W, Wb


def test_noalloc_matches_workspace_entry_twice(B):
    for count, rows, cols in [(4, 1280, 1280), (2, 256, 640)]:
        say(f"muon_update_noalloc count={count} {rows}x{cols}")
        need = B.muon_workspace_size(count, rows, cols)
        assert need <= B.NOALLOC_SCRATCH_BYTES
        ref = _run(B, count, rows, cols, seed=rows + cols, noalloc=False)
        got = _run(B, count, rows, cols, seed=rows + cols, noalloc=True)
        for name, a, b in zip(("O", "M", "W", "W_bf16"), got, ref):
            assert torch.equal(a, b), name
        say(f"  identical to muon_update (scratch {need / 2**20:.1f} MiB of {B.NOALLOC_SCRATCH_BYTES / 2**20:.0f})")


def test_noalloc_rejects_oversized(B):
    """The depth-20 square group needs more scratch than the array holds: the
    host check returns GPT_ERR_WORKSPACE before anything is launched (the
    buffers passed are of the full size all the same)."""
    count, rows, cols = 80, 1280, 1280
    assert B.muon_workspace_size(count, rows, cols) > B.NOALLOC_SCRATCH_BYTES
    G = torch.zeros((count, rows, cols), dtype=torch.float32, device="cuda")
    O = torch.empty_like(G)
    with pytest.raises(B.GptError) as e:
        B.muon_update_noalloc(G, NS5, O_out=O)
    assert e.value.code == -3
    assert "muon_update with a workspace" in str(e.value)
