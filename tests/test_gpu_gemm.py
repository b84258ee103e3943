"""GEMM parity: the HIP bf16 MFMA product against float64 matmul of the same
bf16 values (the definition of a linear layer with bf16 operands)."""

import numpy as np
import pytest
import torch

from gpu_util import bf16_values, from_dev, rel_l2, say, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from gpt_transformer_step_amd import binding
    return binding


def _stored(logical, layout):
    """logical [rows, K] -> the array as stored for that layout, with the
    leading dimension padded to a multiple of 8 elements."""
    st = logical if layout == 0 else logical.T
    ld = (st.shape[1] + 7) // 8 * 8
    out = np.zeros((st.shape[0], ld), dtype=st.dtype)
    out[:, :st.shape[1]] = st
    return out


CASES = [
    # M, N, K, batch, a_layout, b_layout
    (300, 200, 136, 2, 0, 0),
    (300, 200, 136, 2, 0, 1),
    (300, 200, 136, 2, 1, 1),
    (300, 200, 136, 2, 1, 0),
    (8, 8, 8, 1, 0, 0),
    (1024, 768, 512, 1, 0, 0),
    (1024, 768, 512, 1, 0, 1),
    (1024, 768, 520, 1, 1, 1),
    (777, 1030, 64, 1, 0, 0),
    # ragged 256-wide tiles whose K is whole blocks (the block-load loop with
    # clamped rows / chunks), every layout; and ragged 128-wide tiles
    (4992, 1664, 128, 4, 0, 0),
    (4992, 1664, 128, 4, 0, 1),
    (4992, 1664, 128, 4, 1, 0),
    (4992, 1664, 128, 4, 1, 1),
    (1000, 1064, 128, 1, 1, 1),
]


@pytest.mark.parametrize("M,N,K,batch,al,bl", CASES)
@pytest.mark.parametrize("cdt", ["f32", "bf16"])
def test_gemm_layouts(B, M, N, K, batch, al, bl, cdt):
    say(f"gemm M={M} N={N} K={K} batch={batch} layouts=({al},{bl}) C={cdt}")
    g = np.random.default_rng(M * 7 + N + K + al * 2 + bl)
    A = g.standard_normal((batch, M, K)).astype(np.float32)
    Bm = g.standard_normal((batch, N, K)).astype(np.float32)
    As = np.stack([_stored(A[i], al) for i in range(batch)])
    Bs = np.stack([_stored(Bm[i], bl) for i in range(batch)])
    dA, dB = to_dev_bf16(As), to_dev_bf16(Bs)
    tdt = torch.float32 if cdt == "f32" else torch.bfloat16
    ldc = (N + 7) // 8 * 8
    C = torch.zeros((batch, M, ldc), dtype=tdt, device="cuda")
    lda = As.shape[2]
    ldb = Bs.shape[2]
    B.gemm(dA, dB, C, M, N, K, a_layout=al, b_layout=bl, lda=lda, ldb=ldb, ldc=ldc, batch=batch,
           stride_a=As.shape[1] * As.shape[2], stride_b=Bs.shape[1] * Bs.shape[2], stride_c=M * ldc,
           alpha=0.5)
    torch.cuda.synchronize()
    ref = 0.5 * np.einsum("bmk,bnk->bmn", bf16_values(A), bf16_values(Bm))
    got = from_dev(C)
    assert np.all(got[:, :, N:] == 0)  # nothing written past column N
    err = rel_l2(got[:, :, :N], ref)
    tol = 1e-5 if cdt == "f32" else 4e-3
    say(f"  rel_l2 = {err:.3e}")
    assert err < tol


def test_gemm_beta_accumulate(B):
    g = np.random.default_rng(5)
    M, N, K = 260, 132, 72
    A = g.standard_normal((M, K)).astype(np.float32)
    Bm = g.standard_normal((N, K)).astype(np.float32)
    C0 = g.standard_normal((M, N)).astype(np.float32)
    C = torch.from_numpy(C0).cuda()
    B.gemm(to_dev_bf16(A), to_dev_bf16(Bm), C, M, N, K, alpha=1.0, beta=1.0)
    torch.cuda.synchronize()
    ref = C0 + bf16_values(A) @ bf16_values(Bm).T
    assert rel_l2(from_dev(C), ref) < 1e-5


def test_gemm_rejects_bad_args(B):
    A = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    C = torch.zeros(64, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(B.GptError):
        B.gemm(A, A, C, 64, 64, 64, lda=63)
    with pytest.raises(B.GptError):
        B.gemm(A, A, C, 64, 64, 64, a_layout=7)


@pytest.mark.parametrize("M,N,K,al,bl", [
    (65536, 3840, 1280, 0, 0),    # q/k/v projection at depth 20 (32 x 2048 tokens)
    (65536, 1280, 5120, 0, 1),    # MLP data gradient
    (5120, 1280, 65536, 1, 1),    # MLP weight gradient
])
def test_gemm_full_size_sampled(B, M, N, K, al, bl):
    say(f"gemm full size M={M} N={N} K={K} layouts=({al},{bl})")
    g = torch.Generator(device="cuda").manual_seed(3)
    ra = (M, K) if al == 0 else (K, M)
    rb = (N, K) if bl == 0 else (K, N)
    dA = torch.randn(ra, generator=g, device="cuda").to(torch.bfloat16)
    dB = torch.randn(rb, generator=g, device="cuda").to(torch.bfloat16)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    B.gemm(dA, dB, C, M, N, K, a_layout=al, b_layout=bl)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(M, 48, replace=False)
    cols = np.random.default_rng(1).choice(N, 48, replace=False)
    A64 = dA.float().cpu().numpy().astype(np.float64)
    B64 = dB.float().cpu().numpy().astype(np.float64)
    Al = A64 if al == 0 else A64.T
    Bl = B64 if bl == 0 else B64.T
    ref = Al[rows] @ Bl[cols].T
    got = C.cpu().numpy()[np.ix_(rows, cols)]
    err = rel_l2(got, ref)
    say(f"  sampled rel_l2 = {err:.3e}")
    assert err < 1e-5
