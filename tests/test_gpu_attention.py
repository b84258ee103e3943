"""Flash attention parity: gpt_op_attention_fwd / _bwd against the oracle's
plain causal softmax attention on the same bf16 q, k, v (per head)."""

import numpy as np
import pytest
import torch

from gpu_util import bf16_values, cosine, rel_l2, say, to_dev_bf16
from oracle import model as om

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from gpt_transformer_step_amd import binding
    return binding


def _inputs(Bn, H, T, seed, ld_extra=0):
    g = np.random.default_rng(seed)
    d = H * 128
    ld = 3 * d + ld_extra
    # q, k with unit RMS per head (as after the QK normalisation), v ~ N(0,1)
    qkv = g.standard_normal((Bn * T, ld)).astype(np.float32)
    return qkv, ld


def _heads(x, Bn, T, H, off, ld):
    """[B*T, ld] -> [B, H, T, 128] slice starting at column off."""
    return x[:, off: off + H * 128].reshape(Bn, T, H, 128).transpose(0, 2, 1, 3)


@pytest.mark.parametrize("Bn,H,T", [(2, 2, 200), (1, 1, 64), (1, 3, 1), (2, 1, 333), (1, 2, 640)])
def test_attention_fwd_bwd(B, Bn, H, T):
    say(f"attention B={Bn} H={H} T={T}")
    qkv, ld = _inputs(Bn, H, T, seed=Bn * 100 + H * 10 + T)
    d = H * 128
    dq = to_dev_bf16(qkv)
    out = torch.empty((Bn * T, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Bn, H, T), dtype=torch.float32, device="cuda")
    qv = dq.view(torch.int16)
    B.attention_fwd(qv, qv[:, d:], qv[:, 2 * d:], out, lse, Bn, H, T, ld, d)
    torch.cuda.synchronize()
    q64 = bf16_values(qkv).astype(np.float64)
    q, k, v = (_heads(q64, Bn, T, H, o, ld) for o in (0, d, 2 * d))
    y, lse_ref = om.causal_attention(q, k, v)
    y_got = out.float().cpu().numpy().reshape(Bn, T, H, 128).transpose(0, 2, 1, 3)
    e = rel_l2(y_got, y)
    say(f"  out rel_l2 {e:.3e}  lse max err {np.abs(lse.cpu().numpy() - lse_ref).max():.3e}")
    assert e <= 1e-2
    assert np.abs(lse.cpu().numpy() - lse_ref).max() < 1e-3
    # query 0 attends only to key 0: its output is v_0 rounded to bf16
    assert np.array_equal(y_got[:, :, 0], v[:, :, 0])

    g = np.random.default_rng(7)
    dout_np = g.standard_normal((Bn * T, d)).astype(np.float32)
    dout = to_dev_bf16(dout_np)
    delta = torch.empty((Bn, H, T), dtype=torch.float32, device="cuda")
    dq_acc = torch.empty((Bn * T, d), dtype=torch.float32, device="cuda")
    dkv = torch.zeros((Bn * T, ld), dtype=torch.bfloat16, device="cuda")
    dkvv = dkv.view(torch.int16)
    B.attention_bwd(qv, qv[:, d:], qv[:, 2 * d:], out, dout, lse, delta, dq_acc, dkvv[:, d:], dkvv[:, 2 * d:],
                    Bn, H, T, ld, d, ld)
    torch.cuda.synchronize()
    # reference backward on the GPU's own (bf16) output, as the kernel uses it
    y_dev = out.float().cpu().numpy().astype(np.float64).reshape(Bn, T, H, 128).transpose(0, 2, 1, 3)
    dy = bf16_values(dout_np).astype(np.float64).reshape(Bn, T, H, 128).transpose(0, 2, 1, 3)
    dq_r, dk_r, dv_r = om.causal_attention_bwd(q, k, v, y_dev, dy, lse_ref)
    dq_g = dq_acc.cpu().numpy().reshape(Bn, T, H, 128).transpose(0, 2, 1, 3)
    dkv_np = dkv.float().cpu().numpy()
    dk_g = _heads(dkv_np, Bn, T, H, d, ld)
    dv_g = _heads(dkv_np, Bn, T, H, 2 * d, ld)
    for name, got, ref in (("dq", dq_g, dq_r), ("dk", dk_g, dk_r), ("dv", dv_g, dv_r)):
        e, c = rel_l2(got, ref), cosine(got, ref)
        say(f"  {name} rel_l2 {e:.3e} cos {c:.6f}")
        assert e <= 1e-2 and c >= 0.999


def test_attention_full_size_sampled(B):
    """depth-20 shape (32 sequences x 10 heads x 2048), forward and backward
    as the step launches them: the oracle checks sampled (sequence, head)
    pairs (out and lse; dq, dk, dv); every output is checked finite."""
    Bn, H, T = 32, 10, 2048
    d = H * 128
    say(f"attention full size B={Bn} H={H} T={T}")
    gen = torch.Generator(device="cuda").manual_seed(11)
    qkv = torch.randn((Bn * T, 3 * d), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((Bn * T, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Bn, H, T), dtype=torch.float32, device="cuda")
    qv = qkv.view(torch.int16)
    B.attention_fwd(qv, qv[:, d:], qv[:, 2 * d:], out, lse, Bn, H, T, 3 * d, d)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    for (b, h) in [(0, 0), (31, 9)]:
        rows = qkv[b * T:(b + 1) * T].float().cpu().numpy().astype(np.float64)
        q = rows[:, h * 128:(h + 1) * 128]
        k = rows[:, d + h * 128: d + (h + 1) * 128]
        v = rows[:, 2 * d + h * 128: 2 * d + (h + 1) * 128]
        y, l = om.causal_attention(q, k, v)
        got = out[b * T:(b + 1) * T, h * 128:(h + 1) * 128].float().cpu().numpy()
        e = rel_l2(got, y)
        say(f"  (b={b}, h={h}) out rel_l2 {e:.3e}")
        assert e <= 1e-2
        assert np.abs(lse[b, h].cpu().numpy() - l).max() < 1e-3

    gen.manual_seed(12)
    dout = torch.randn((Bn * T, d), generator=gen, device="cuda").to(torch.bfloat16)
    delta = torch.empty((Bn, H, T), dtype=torch.float32, device="cuda")
    dq_acc = torch.empty((Bn * T, d), dtype=torch.float32, device="cuda")
    dkv = torch.zeros((Bn * T, 3 * d), dtype=torch.bfloat16, device="cuda")
    dkvv = dkv.view(torch.int16)
    B.attention_bwd(qv, qv[:, d:], qv[:, 2 * d:], out, dout, lse, delta, dq_acc, dkvv[:, d:], dkvv[:, 2 * d:],
                    Bn, H, T, 3 * d, d, 3 * d)
    torch.cuda.synchronize()
    assert torch.isfinite(dq_acc).all() and torch.isfinite(dkv.float()).all()
    for (b, h) in [(0, 0), (13, 4), (31, 9)]:
        rows = qkv[b * T:(b + 1) * T].float().cpu().numpy().astype(np.float64)
        q, k, v = (rows[:, o + h * 128: o + (h + 1) * 128][None, None] for o in (0, d, 2 * d))
        # reference backward on the GPU's own (bf16) output, as the kernels use it
        y_dev = out[b * T:(b + 1) * T, h * 128:(h + 1) * 128].float().cpu().numpy().astype(np.float64)[None, None]
        dy = dout[b * T:(b + 1) * T, h * 128:(h + 1) * 128].float().cpu().numpy().astype(np.float64)[None, None]
        _, l_ref = om.causal_attention(q, k, v)
        dq_r, dk_r, dv_r = om.causal_attention_bwd(q, k, v, y_dev, dy, l_ref)
        got = {"dq": dq_acc[b * T:(b + 1) * T, h * 128:(h + 1) * 128],
               "dk": dkv[b * T:(b + 1) * T, d + h * 128: d + (h + 1) * 128],
               "dv": dkv[b * T:(b + 1) * T, 2 * d + h * 128: 2 * d + (h + 1) * 128]}
        for name, ref in (("dq", dq_r), ("dk", dk_r), ("dv", dv_r)):
            g_np = got[name].float().cpu().numpy()
            e, c = rel_l2(g_np, ref[0, 0]), cosine(g_np, ref[0, 0])
            say(f"  (b={b}, h={h}) {name} rel_l2 {e:.3e} cos {c:.6f}")
            assert e <= 1e-2 and c >= 0.999


@pytest.mark.parametrize("Bn,H,Hkv,T,window", [
    (2, 4, 2, 200, 37),      # grouped heads, window shorter than a tile, ragged T
    (1, 4, 1, 333, 64),      # one shared key/value head, window = one key tile
    (1, 2, 2, 640, 200),     # plain heads, window spanning several tiles
    (2, 2, 1, 150, -1),      # grouped heads, full causal
    (1, 1, 1, 70, 0),        # window 0: every query sees only its own key
])
def test_attention_gqa_window(B, Bn, H, Hkv, T, window):
    """Query head h reads key/value head h / (H / Hkv); with window w >= 0,
    query i sees keys i - w .. i.  The oracle repeats each key/value head over
    its group and applies the window mask; dK and dV of a shared head are the
    sums over the query heads of its group."""
    say(f"attention GQA/window B={Bn} H={H} Hkv={Hkv} T={T} window={window}")
    d, dkv = H * 128, Hkv * 128
    ld = d + 2 * dkv
    g = np.random.default_rng(Bn * 1000 + H * 100 + Hkv * 10 + T + window)
    qkv = g.standard_normal((Bn * T, ld)).astype(np.float32)
    dq = to_dev_bf16(qkv)
    qv = dq.view(torch.int16)
    out = torch.empty((Bn * T, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Bn, H, T), dtype=torch.float32, device="cuda")
    B.attention_fwd(qv, qv[:, d:], qv[:, d + dkv:], out, lse, Bn, H, T, ld, d, n_kv_head=Hkv, window=window)
    torch.cuda.synchronize()
    grp = H // Hkv
    w = None if window < 0 else window
    x64 = bf16_values(qkv).astype(np.float64)
    q = _heads(x64, Bn, T, H, 0, ld)
    k = np.repeat(_heads(x64, Bn, T, Hkv, d, ld), grp, axis=1)
    v = np.repeat(_heads(x64, Bn, T, Hkv, d + dkv, ld), grp, axis=1)
    y, lse_ref = om.causal_attention(q, k, v, window=w)
    y_got = out.float().cpu().numpy().reshape(Bn, T, H, 128).transpose(0, 2, 1, 3)
    e = rel_l2(y_got, y)
    say(f"  out rel_l2 {e:.3e}  lse max err {np.abs(lse.cpu().numpy() - lse_ref).max():.3e}")
    assert e <= 1e-2
    assert np.abs(lse.cpu().numpy() - lse_ref).max() < 1e-3
    if window == 0:
        # softmax over a single key: the output is v_i itself (bf16)
        assert np.array_equal(y_got, v)

    dout_np = g.standard_normal((Bn * T, d)).astype(np.float32)
    dout = to_dev_bf16(dout_np)
    delta = torch.empty((Bn, H, T), dtype=torch.float32, device="cuda")
    dq_acc = torch.empty((Bn * T, d), dtype=torch.float32, device="cuda")
    dkv_t = torch.zeros((Bn * T, ld), dtype=torch.bfloat16, device="cuda")
    dkvv = dkv_t.view(torch.int16)
    B.attention_bwd(qv, qv[:, d:], qv[:, d + dkv:], out, dout, lse, delta, dq_acc, dkvv[:, d:],
                    dkvv[:, d + dkv:], Bn, H, T, ld, d, ld, n_kv_head=Hkv, window=window)
    torch.cuda.synchronize()
    y_dev = out.float().cpu().numpy().astype(np.float64).reshape(Bn, T, H, 128).transpose(0, 2, 1, 3)
    dy = bf16_values(dout_np).astype(np.float64).reshape(Bn, T, H, 128).transpose(0, 2, 1, 3)
    dq_r, dk_r, dv_r = om.causal_attention_bwd(q, k, v, y_dev, dy, lse_ref, window=w)
    dk_r = dk_r.reshape(Bn, Hkv, grp, T, 128).sum(axis=2)
    dv_r = dv_r.reshape(Bn, Hkv, grp, T, 128).sum(axis=2)
    dq_g = dq_acc.cpu().numpy().reshape(Bn, T, H, 128).transpose(0, 2, 1, 3)
    dkv_np = dkv_t.float().cpu().numpy()
    dk_g = _heads(dkv_np, Bn, T, Hkv, d, ld)
    dv_g = _heads(dkv_np, Bn, T, Hkv, d + dkv, ld)
    checks = (("dq", dq_g, dq_r), ("dk", dk_g, dk_r), ("dv", dv_g, dv_r))
    if window == 0:
        # P = 1 on the diagonal: dS = dP - rowsum(dY * Y) = 0 exactly, so dQ and
        # dK are rounding noise on both sides; only dV = dY has a definite value
        for name, got in (("dq", dq_g), ("dk", dk_g)):
            say(f"  {name} max |.| {np.abs(got).max():.3e}")
            assert np.abs(got).max() <= 1e-3
        checks = checks[2:]
    for name, got, ref in checks:
        e, c = rel_l2(got, ref), cosine(got, ref)
        say(f"  {name} rel_l2 {e:.3e} cos {c:.6f}")
        assert e <= 1e-2 and c >= 0.999
