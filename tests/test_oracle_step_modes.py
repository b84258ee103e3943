"""Pins of the oracle's two reduced-precision step modes against an
independent torch CPU implementation of the tiny model.

fp8 mode (precision passage: apidog.com/pt "Gerenciamento de Precisão",
apidog.com/de "Präzisionsverwaltung" -- linear layers in fp8 with one scale per
tensor): torch autograd in float64 with each block product (the fused q/k/v
weight as one tensor, the output projection, fc and proj) replaced by a
custom function built on torch's own float8_e4m3fn / float8_e5m2 casts
(clamped first, scale = fmax / amax in fp32): forward Q43(X) Q43(W)^T, data
gradient Q52(dY) Q43(W), weight gradient Q52(dY)^T Q43(X).  None of
oracle/fp8.py is used.  The oracle's fp8 mode must match it to 1e-12.

bf16 mode (dev.to "3. Gestión de Precisión": products in the bf16 compute
dtype): with the rounding replaced by a recorder, the oracle must round
exactly the documented tensors, in order -- each recorded tensor is compared
with the matching intermediate (or its gradient) of a torch autograd run of
the same model with the softmax written out.
"""

import math

import numpy as np
import pytest

from oracle import model as om

torch = pytest.importorskip("torch")
F = torch.nn.functional

TINY = om.Config(n_layer=2, d_model=16, n_head=2, head_dim=8, hidden=64, vocab=37)


def _params(cfg, seed, scale=1.5):
    g = np.random.default_rng(seed)
    return {n: g.standard_normal(s) * scale / math.sqrt(s[1]) for n, s in om.param_shapes(cfg).items()}


def _ids(cfg, B, T, seed):
    return np.random.default_rng(seed).integers(0, cfg.vocab, size=(B, T + 1))


def _q(t, tdt, fmax):
    """Per-tensor fake quantisation with torch's cast: s = fmax / amax (fp32),
    value = cast(clamp(t * s)) / s."""
    amax = t.detach().abs().max().to(torch.float32)
    s = torch.tensor(fmax, dtype=torch.float32) / amax if amax > 0 else torch.tensor(1.0, dtype=torch.float32)
    scaled = (t.detach().to(torch.float32) * s).clamp(-fmax, fmax)
    return scaled.to(tdt).to(torch.float64) / s.to(torch.float64)


def q43(t):
    return _q(t, torch.float8_e4m3fn, 448.0)


def q52(t):
    return _q(t, torch.float8_e5m2, 57344.0)


class Fp8Linear(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w):
        ctx.save_for_backward(x, w)
        return q43(x) @ q43(w).T

    @staticmethod
    def backward(ctx, dy):
        x, w = ctx.saved_tensors
        g = q52(dy)
        return g @ q43(w), g.T @ q43(x)


def _torch_model(cfg, P, ids, lin, record=None):
    """Forward of the tiny model in torch float64; lin(x, w) is the block
    product; record (dict) receives the intermediates whose gradients are
    kept."""
    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in P.items()}
    B, T = ids.shape[0], ids.shape[1] - 1
    d, H, hd = cfg.d_model, cfg.n_head, cfg.head_dim
    inp, tgt = torch.tensor(ids[:, :T]), torch.tensor(ids[:, 1:])
    ang = torch.arange(T, dtype=torch.float64)[:, None] * cfg.rope_base ** (
        -torch.arange(0, hd, 2, dtype=torch.float64) / hd)[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)

    def rope_t(x):
        xc = torch.complex(x[..., : hd // 2], x[..., hd // 2:]) * rot
        return torch.cat([xc.real, xc.imag], dim=-1)

    def rms(x, n):
        return F.rms_norm(x, (n,), eps=cfg.eps)

    def keep(name, t):
        if record is not None:
            t.retain_grad()
            record[name] = t
        return t

    mask = torch.triu(torch.ones(T, T, dtype=torch.bool), 1)
    x = tp["wte"][inp].reshape(B * T, d)
    for i in range(cfg.n_layer):
        h = keep(f"h1.{i}", rms(x, d))
        wqkv = torch.cat([tp[f"wq.{i}"], tp[f"wk.{i}"], tp[f"wv.{i}"]], 0)
        qkv = keep(f"qkv.{i}", lin(h, wqkv))
        q = qkv[:, :d].reshape(B, T, H, hd).transpose(1, 2)
        k = qkv[:, d:2 * d].reshape(B, T, H, hd).transpose(1, 2)
        v = keep(f"v.{i}", qkv[:, 2 * d:].reshape(B, T, H, hd).transpose(1, 2))
        q = keep(f"q.{i}", rms(rope_t(q), hd))
        k = keep(f"k.{i}", rms(rope_t(k), hd))
        s = keep(f"s.{i}", (q @ k.transpose(-1, -2) / math.sqrt(hd)).masked_fill(mask, -math.inf))
        p = keep(f"p.{i}", torch.softmax(s, -1))
        y = keep(f"y.{i}", (p @ v).transpose(1, 2).reshape(B * T, d))
        x = keep(f"xa.{i}", x + lin(y, tp[f"wo.{i}"]))
        h2 = keep(f"h2.{i}", rms(x, d))
        u = keep(f"u.{i}", lin(h2, tp[f"wfc.{i}"]))
        a = keep(f"a.{i}", F.relu(u).square())
        x = keep(f"xm.{i}", x + lin(a, tp[f"wproj.{i}"]))
    hf = keep("hf", rms(x, d))
    z = keep("z", hf @ tp["lm_head"].T)
    loss = F.cross_entropy(z, tgt.reshape(-1))
    loss.backward()
    return loss, tp


def test_fp8_mode_matches_torch_float8_casts():
    cfg = TINY
    P = _params(cfg, seed=51)
    ids = _ids(cfg, B=3, T=8, seed=52)
    out = om.forward_backward(P, ids, cfg, fp8=True)
    loss, tp = _torch_model(cfg, P, ids, Fp8Linear.apply)
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-12)
    for name in om.param_names(cfg):
        ref = tp[name].grad.numpy()
        got = out["grads"][name]
        assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max()), name
    # the quantisation is active: the fp8 mode differs from the exact one
    exact = om.forward_backward(P, ids, cfg)
    assert abs(exact["loss"] - out["loss"]) > 1e-6


def test_bf16_mode_rounds_exactly_the_documented_tensors(monkeypatch):
    cfg = TINY
    P = _params(cfg, seed=61)
    ids = _ids(cfg, B=2, T=8, seed=62)
    rec = {}
    loss, _ = _torch_model(cfg, P, ids, lambda x, w: x @ w.T, record=rec)
    seen = []
    from oracle import precision

    def recorder(t):
        seen.append(np.array(t, dtype=np.float64))
        return np.asarray(t)

    monkeypatch.setattr(precision, "round_bf16", recorder)
    out = om.forward_backward(P, ids, cfg, bf16_operands=True)
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-12)

    def val(name):
        return rec[name].detach()

    def grad(name):
        return rec[name].grad.detach()

    want = []
    for i in range(cfg.n_layer):
        want += [("h1", val(f"h1.{i}")), ("v", val(f"v.{i}")), ("q", val(f"q.{i}")), ("k", val(f"k.{i}")),
                 ("P", val(f"p.{i}")), ("y", val(f"y.{i}")), ("h2", val(f"h2.{i}")), ("a", val(f"a.{i}"))]
    want += [("hf", val("hf")), ("dz", grad("z")), ("dhf", grad("hf"))]
    for i in reversed(range(cfg.n_layer)):
        dqkv = grad(f"qkv.{i}")
        want += [("g mlp", grad(f"xm.{i}")), ("du", grad(f"u.{i}")), ("dh2", grad(f"h2.{i}")),
                 ("g attn", grad(f"xa.{i}")), ("dO", grad(f"y.{i}")), ("P bwd", val(f"p.{i}")),
                 ("dS", grad(f"s.{i}").nan_to_num(0.0)), ("dqkv", dqkv), ("dh1", grad(f"h1.{i}"))]
    assert len(seen) == len(want), [w[0] for w in want]
    for j, ((name, ref), got) in enumerate(zip(want, seen)):
        ref = ref.numpy()
        if name in ("P", "P bwd", "dS"):
            ref = np.where(np.isfinite(ref), ref, 0.0)
        assert got.shape == ref.shape, (j, name, got.shape, ref.shape)
        err = np.abs(got - ref).max()
        assert err <= 1e-11 * max(1.0, np.abs(ref).max()), (j, name, err)


def test_jitter_seed_is_a_bf16_computation():
    """A jitter seed gives another bf16 computation of the step: deterministic
    per seed, different between seeds, and as far from the exact step as the
    unjittered bf16 mode (a fp32-sized perturbation only reshuffles which
    values round up)."""
    cfg = TINY
    P = _params(cfg, seed=71)
    ids = _ids(cfg, B=2, T=8, seed=72)
    ex = om.forward_backward(P, ids, cfg)
    b0 = om.forward_backward(P, ids, cfg, bf16_operands=True)
    j1 = om.forward_backward(P, ids, cfg, bf16_operands=True, jitter_seed=1)
    j1b = om.forward_backward(P, ids, cfg, bf16_operands=True, jitter_seed=1)
    j2 = om.forward_backward(P, ids, cfg, bf16_operands=True, jitter_seed=2)
    assert j1["loss"] == j1b["loss"]
    assert any(not np.array_equal(j1["grads"][n], j2["grads"][n]) for n in j1["grads"])
    for n in ex["grads"]:
        e0 = np.linalg.norm(b0["grads"][n] - ex["grads"][n])
        for j in (j1, j2):
            e = np.linalg.norm(j["grads"][n] - ex["grads"][n])
            assert e <= 3.0 * e0 + 1e-3 * np.linalg.norm(ex["grads"][n]), n
    with pytest.raises(ValueError):
        om.forward_backward(P, ids, cfg, jitter_seed=1)
