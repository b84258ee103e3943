"""Pins of the oracle's forward/backward against things other than itself.

* central finite differences (float64) of the loss for sampled entries of every
  parameter tensor on a tiny shape;
* a brute-force double loop for causal attention;
* torch CPU autograd (float64) with torch's RMS norm, scaled-dot-product
  attention and cross-entropy as a second, independent implementation;
* closed forms: zero output matrix -> loss = ln V; attention rows sum to 1
  and row 0 returns v_0; RMSNorm mean square; RoPE identity, norm and
  relative-position properties.
"""

import math

import numpy as np
import pytest

from oracle import model as om
from gpt_transformer_step_amd import inputs

TINY = om.Config(n_layer=2, d_model=16, n_head=2, head_dim=8, hidden=64, vocab=37)


def _tiny_params(cfg, seed=0, scale=1.0):
    g = np.random.default_rng(seed)
    P = {}
    for name, shape in om.param_shapes(cfg).items():
        P[name] = g.standard_normal(shape) * scale / math.sqrt(shape[1])
    return P


def _tiny_ids(cfg, B=2, T=8, seed=1):
    return np.random.default_rng(seed).integers(0, cfg.vocab, size=(B, T + 1))


def test_finite_differences_every_tensor():
    cfg = TINY
    P = _tiny_params(cfg, scale=2.0)
    ids = _tiny_ids(cfg)
    out = om.forward_backward(P, ids, cfg)
    rng = np.random.default_rng(7)
    h = 1e-5
    worst = 0.0
    for name in om.param_names(cfg):
        W = P[name]
        for _ in range(4):
            idx = tuple(int(rng.integers(0, s)) for s in W.shape)
            if name == "wte":  # pick a row that is used, else the gradient is exactly 0
                idx = (int(ids[0, int(rng.integers(0, ids.shape[1] - 1))]), idx[1])
            old = W[idx]
            W[idx] = old + h
            lp = om.forward_backward(P, ids, cfg, want_grads=False)["loss"]
            W[idx] = old - h
            lm = om.forward_backward(P, ids, cfg, want_grads=False)["loss"]
            W[idx] = old
            fd = (lp - lm) / (2 * h)
            an = out["grads"][name][idx]
            # central differences: truncation ~h^2, round-off ~1e-16 * loss / h
            err = abs(fd - an) / (abs(an) + 1e-4)
            worst = max(worst, err)
            assert err < 1e-6, (name, idx, fd, an)
    assert worst < 1e-6


def test_lm_head_zero_gives_ln_vocab():
    cfg = TINY
    P = _tiny_params(cfg)
    P["lm_head"][:] = 0.0
    ids = _tiny_ids(cfg)
    out = om.forward_backward(P, ids, cfg)
    assert out["loss"] == pytest.approx(math.log(cfg.vocab), abs=1e-14)
    # with zero logits dz = (1/V - onehot)/N, so dW_lm = dz^T h_f has rows
    # that sum (over vocab) to zero
    assert np.abs(out["grads"]["lm_head"].sum(axis=0)).max() < 1e-12


def test_full_vocab_ln():
    # the full configuration's vocabulary: ln 32768 exactly when the head is 0
    z = np.zeros((3, 32768))
    loss, lse = om.cross_entropy(z, np.array([0, 5, 32767]))
    assert np.allclose(loss, 10.397207708399179, atol=1e-12)


def test_attention_bruteforce_and_rows():
    g = np.random.default_rng(3)
    H, T, hd = 2, 9, 8
    q, k, v = (g.standard_normal((H, T, hd)) for _ in range(3))
    y, lse = om.causal_attention(q, k, v)
    for h in range(H):
        for i in range(T):
            s = [float(np.dot(q[h, i], k[h, j])) / math.sqrt(hd) for j in range(i + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            den = sum(w)
            ref = sum(w[j] / den * v[h, j] for j in range(i + 1))
            assert np.allclose(y[h, i], ref, atol=1e-13)
            assert lse[h, i] == pytest.approx(m + math.log(den), abs=1e-13)
    # rows of P sum to one: with v all ones the output is all ones
    y1, _ = om.causal_attention(q, k, np.ones_like(v))
    assert np.abs(y1 - 1).max() < 1e-13
    # query 0 sees only key 0
    assert np.array_equal(y[:, 0], v[:, 0])


def test_rms_norm_mean_square():
    g = np.random.default_rng(4)
    x = g.standard_normal((5, 64)) * 3
    y, r = om.rms_norm(x, 1e-6)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + 1e-6), rtol=1e-13)


def test_rope_properties():
    T, hd = 16, 8
    cos, sin = om.rope_tables(T, hd, 10000.0)
    g = np.random.default_rng(5)
    q = g.standard_normal((T, hd))
    k = g.standard_normal((T, hd))
    rq = om.rope(q, cos, sin)
    # position 0 is the identity
    assert np.array_equal(rq[0], q[0])
    # rotation keeps the norm
    assert np.allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-13)
    # <R_m a, R_n b> depends only on m - n
    a, b = q[0], k[0]
    A = om.rope(np.tile(a, (T, 1)), cos, sin)
    Bv = om.rope(np.tile(b, (T, 1)), cos, sin)
    assert np.dot(A[7], Bv[3]) == pytest.approx(np.dot(A[4], Bv[0]), abs=1e-12)
    assert np.dot(A[9], Bv[9]) == pytest.approx(np.dot(a, b), abs=1e-12)
    # the backward is the inverse rotation
    assert np.allclose(om.rope_bwd(rq, cos, sin), q, atol=1e-13)
    # the gainless RMS norm commutes with the rotation
    n1, _ = om.rms_norm(om.rope(q, cos, sin), 1e-6)
    n2 = om.rope(om.rms_norm(q, 1e-6)[0], cos, sin)
    assert np.allclose(n1, n2, atol=1e-13)


def test_against_torch_autograd():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    cfg = TINY
    P = _tiny_params(cfg, seed=11, scale=1.5)
    ids = _tiny_ids(cfg, B=3, T=8, seed=12)
    out = om.forward_backward(P, ids, cfg)

    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in P.items()}
    B, T = ids.shape[0], ids.shape[1] - 1
    d, H, hd = cfg.d_model, cfg.n_head, cfg.head_dim
    inp = torch.tensor(ids[:, :T])
    tgt = torch.tensor(ids[:, 1:])
    pos = torch.arange(T, dtype=torch.float64)
    freq = cfg.rope_base ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = pos[:, None] * freq[None, :]
    # complex-number form of the rotation: (x1 + i x2) * e^{i theta}
    rot = torch.polar(torch.ones_like(ang), ang)

    def rope_t(x):  # x [B, H, T, hd]
        xc = torch.complex(x[..., : hd // 2], x[..., hd // 2:]) * rot
        return torch.cat([xc.real, xc.imag], dim=-1)

    def rms(x, n):
        return F.rms_norm(x, (n,), eps=cfg.eps)

    x = tp["wte"][inp]
    for i in range(cfg.n_layer):
        h = rms(x, d)
        q = (h @ tp[f"wq.{i}"].T).view(B, T, H, hd).transpose(1, 2)
        k = (h @ tp[f"wk.{i}"].T).view(B, T, H, hd).transpose(1, 2)
        v = (h @ tp[f"wv.{i}"].T).view(B, T, H, hd).transpose(1, 2)
        q = rms(rope_t(q), hd)
        k = rms(rope_t(k), hd)
        y = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        x = x + y.transpose(1, 2).reshape(B, T, d) @ tp[f"wo.{i}"].T
        h = rms(x, d)
        x = x + F.relu(h @ tp[f"wfc.{i}"].T).square() @ tp[f"wproj.{i}"].T
    z = rms(x, d) @ tp["lm_head"].T
    loss = F.cross_entropy(z.reshape(-1, cfg.vocab), tgt.reshape(-1))
    loss.backward()
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-12)
    for name in om.param_names(cfg):
        ref = tp[name].grad.numpy()
        got = out["grads"][name]
        assert np.abs(got - ref).max() <= 1e-11 * max(1.0, np.abs(ref).max()), name


def test_seq_chunking_matches_whole_batch():
    cfg = TINY
    P = _tiny_params(cfg, seed=21)
    ids = _tiny_ids(cfg, B=4, T=8, seed=22)
    a = om.forward_backward(P, ids, cfg)
    b = om.forward_backward(P, ids, cfg, seq_chunk=1)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-13)
    for k in a["grads"]:
        assert np.allclose(a["grads"][k], b["grads"][k], rtol=1e-12, atol=1e-15)


def test_gather_and_targets_are_exact():
    # the inputs are ids[:, :T] gathered from wte; the targets are ids[:, 1:]
    cfg = TINY
    P = _tiny_params(cfg, seed=31)
    ids = _tiny_ids(cfg, B=2, T=8, seed=32)
    out = om.forward_backward(P, ids, cfg, want_grads=False, want_logits=True)
    z = out["logits"]
    tgt = ids[:, 1:].reshape(-1)
    assert np.allclose(out["row_loss"].reshape(-1), out["lse"].reshape(-1) - z[np.arange(len(tgt)), tgt])


def test_inputs_generator_is_stable():
    dims = inputs.Dims.from_depth(2)
    ids = inputs.token_ids(2, 128, 32768, inputs.SEED_IDS)
    assert ids.shape == (2, 129) and ids.dtype == np.int32
    assert ids.min() >= 0 and ids.max() < 32768
    w = inputs.master_weights(dims, inputs.SEED_W)
    assert w.shape == (inputs.n_params(dims),)
    w2 = inputs.master_weights(dims, inputs.SEED_W)
    assert inputs.sha256(w) == inputs.sha256(w2)
    t = inputs.unpack(dims, w)
    # std close to 1/sqrt(fan_in)
    assert abs(t["wfc.0"].std() * math.sqrt(128) - 1) < 0.02
    assert abs(t["wproj.1"].std() * math.sqrt(512) - 1) < 0.02


def test_bf16_operand_mode():
    """The bf16-operand reading changes only the rounding of product operands:
    with weights and data that are already bf16-exact at every operand point
    it is identical to the exact mode, and otherwise it stays within bf16
    rounding distance of it."""
    cfg = TINY
    P = _tiny_params(cfg, seed=41)
    ids = _tiny_ids(cfg, B=2, T=8, seed=42)
    a = om.forward_backward(P, ids, cfg)
    b = om.forward_backward(P, ids, cfg, bf16_operands=True)
    assert abs(a["loss"] - b["loss"]) < 1e-2 * abs(a["loss"])
    for k in a["grads"]:
        num = np.linalg.norm(a["grads"][k] - b["grads"][k])
        assert num <= 5e-2 * np.linalg.norm(a["grads"][k]) + 1e-12, k
        # the modes really differ (the rounding is applied)
    assert any(not np.array_equal(a["grads"][k], b["grads"][k]) for k in a["grads"])


def test_bf16_operand_rounding_points(monkeypatch):
    """Every rounding the mode applies is to an operand of a matrix product:
    replacing the rounding by the identity gives back the exact mode bit for bit."""
    cfg = TINY
    P = _tiny_params(cfg, seed=43)
    ids = _tiny_ids(cfg, B=2, T=8, seed=44)
    a = om.forward_backward(P, ids, cfg)
    from oracle import precision
    monkeypatch.setattr(precision, "round_bf16", lambda t: np.asarray(t))
    b = om.forward_backward(P, ids, cfg, bf16_operands=True)
    assert a["loss"] == b["loss"]
    for k in a["grads"]:
        assert np.array_equal(a["grads"][k], b["grads"][k])


# ---------------------------------------------------------------------------
# grouped key/value heads (GQA) and sliding-window layers
# ---------------------------------------------------------------------------
TINY_GQA = om.Config(n_layer=3, d_model=32, n_head=4, head_dim=8, hidden=64, vocab=29,
                     n_kv_head=2, window=3, pattern="SL")


def test_window_attention_bruteforce():
    g = np.random.default_rng(13)
    H, T, hd, w = 2, 11, 8, 3
    q, k, v = (g.standard_normal((H, T, hd)) for _ in range(3))
    y, lse = om.causal_attention(q, k, v, window=w)
    for h in range(H):
        for i in range(T):
            js = [j for j in range(T) if i - w <= j <= i]
            s = [float(np.dot(q[h, i], k[h, j])) / math.sqrt(hd) for j in js]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            den = sum(e)
            ref = sum(e[n] / den * v[h, j] for n, j in enumerate(js))
            assert np.allclose(y[h, i], ref, atol=1e-13)
            assert lse[h, i] == pytest.approx(m + math.log(den), abs=1e-13)
    # a window as long as the sequence is the full causal mask
    y_full, _ = om.causal_attention(q, k, v)
    y_wide, _ = om.causal_attention(q, k, v, window=T)
    assert np.array_equal(y_full, y_wide)


def test_layer_window_pattern():
    cfg = TINY_GQA
    assert [cfg.layer_window(i) for i in range(4)] == [3, None, 3, None]
    assert om.Config.from_depth(4, 100, window=64, pattern="SSSL").layer_window(3) is None
    assert om.Config.from_depth(4, 100, window=64, pattern="SSSL").layer_window(5) == 64
    assert om.Config.from_depth(4, 100).layer_window(0) is None
    shapes = om.param_shapes(cfg)
    assert shapes["wk.0"] == (16, 32) and shapes["wv.2"] == (16, 32) and shapes["wq.1"] == (32, 32)


def test_finite_differences_gqa_window():
    cfg = TINY_GQA
    P = _tiny_params(cfg, seed=51, scale=2.0)
    ids = _tiny_ids(cfg, B=2, T=9, seed=52)
    out = om.forward_backward(P, ids, cfg)
    rng = np.random.default_rng(53)
    h = 1e-5
    for name in om.param_names(cfg):
        W = P[name]
        for _ in range(3):
            idx = tuple(int(rng.integers(0, s)) for s in W.shape)
            if name == "wte":
                idx = (int(ids[0, int(rng.integers(0, ids.shape[1] - 1))]), idx[1])
            old = W[idx]
            W[idx] = old + h
            lp = om.forward_backward(P, ids, cfg, want_grads=False)["loss"]
            W[idx] = old - h
            lm = om.forward_backward(P, ids, cfg, want_grads=False)["loss"]
            W[idx] = old
            fd = (lp - lm) / (2 * h)
            an = out["grads"][name][idx]
            assert abs(fd - an) / (abs(an) + 1e-4) < 1e-6, (name, idx, fd, an)


def test_gqa_window_against_torch_autograd():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    cfg = TINY_GQA
    P = _tiny_params(cfg, seed=61, scale=1.5)
    ids = _tiny_ids(cfg, B=2, T=10, seed=62)
    out = om.forward_backward(P, ids, cfg)
    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in P.items()}
    B, T = ids.shape[0], ids.shape[1] - 1
    d, H, Hkv, hd = cfg.d_model, cfg.n_head, cfg.n_kv_head, cfg.head_dim
    inp, tgt = torch.tensor(ids[:, :T]), torch.tensor(ids[:, 1:])
    freq = cfg.rope_base ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    rot = torch.polar(torch.ones(T, hd // 2, dtype=torch.float64),
                      torch.arange(T, dtype=torch.float64)[:, None] * freq[None, :])

    def rope_t(x):
        xc = torch.complex(x[..., : hd // 2], x[..., hd // 2:]) * rot
        return torch.cat([xc.real, xc.imag], dim=-1)

    def rms(x, n):
        return F.rms_norm(x, (n,), eps=cfg.eps)

    ii = torch.arange(T)[:, None]
    jj = torch.arange(T)[None, :]
    x = tp["wte"][inp]
    for i in range(cfg.n_layer):
        h = rms(x, d)
        q = (h @ tp[f"wq.{i}"].T).view(B, T, H, hd).transpose(1, 2)
        k = (h @ tp[f"wk.{i}"].T).view(B, T, Hkv, hd).transpose(1, 2)
        v = (h @ tp[f"wv.{i}"].T).view(B, T, Hkv, hd).transpose(1, 2)
        q, k = rms(rope_t(q), hd), rms(rope_t(k), hd)
        w = cfg.layer_window(i)
        allowed = jj <= ii if w is None else (jj <= ii) & (jj >= ii - w)
        y = F.scaled_dot_product_attention(q, k.repeat_interleave(H // Hkv, dim=1),
                                           v.repeat_interleave(H // Hkv, dim=1), attn_mask=allowed)
        x = x + y.transpose(1, 2).reshape(B, T, d) @ tp[f"wo.{i}"].T
        h = rms(x, d)
        x = x + F.relu(h @ tp[f"wfc.{i}"].T).square() @ tp[f"wproj.{i}"].T
    z = rms(x, d) @ tp["lm_head"].T
    loss = F.cross_entropy(z.reshape(-1, cfg.vocab), tgt.reshape(-1))
    loss.backward()
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-12)
    for name in om.param_names(cfg):
        ref = tp[name].grad.numpy()
        assert np.abs(out["grads"][name] - ref).max() <= 1e-11 * max(1.0, np.abs(ref).max()), name


def test_inputs_gqa_shapes():
    dims = inputs.Dims.from_depth(4, 1000, n_kv_head=1)
    shp = dict(inputs.packed_tensors(dims))
    assert shp["wk.0"] == (128, 256) and shp["wv.3"] == (128, 256) and shp["wq.0"] == (256, 256)
    assert inputs.Dims.from_depth(4).d_kv == 256


# ---------------------------------------------------------------------------
# record-model features: value embeddings, smear, residual scaling, backout
# ---------------------------------------------------------------------------

TINY_FEAT = om.Config(n_layer=4, d_model=48, n_head=6, head_dim=8, hidden=96, vocab=31, n_kv_head=3,
                      window=3, pattern="SL", value_embeds=True, smear=True, resid_lambdas=True, backout=True)


def _feat_params(cfg, seed=0, scale=1.5):
    """Matrices N(0, scale^2 / fan_in); scalars near their neutral values."""
    g = np.random.default_rng(seed)
    P = {}
    for name, shape in om.param_shapes(cfg).items():
        z = g.standard_normal(shape)
        if name == "resid_lambda":
            P[name] = 1.0 + 0.2 * z
        elif name == "x0_lambda":
            P[name] = 0.3 * z
        elif name == "smear_lambda":
            P[name] = 0.6 + 0.2 * z
        elif name == "backout_lambda":
            P[name] = 0.3 + 0.1 * z
        else:
            P[name] = z * scale / math.sqrt(shape[-1])
    return P


def test_feature_layout():
    cfg = TINY_FEAT
    names = om.param_names(cfg)
    assert names[-5:] == ["resid_lambda", "x0_lambda", "smear_w", "smear_lambda", "backout_lambda"]
    assert [n for n in names if n.startswith("ve.")] == ["ve.0", "ve.2"]
    shp = om.param_shapes(cfg)
    assert shp["ve.2"] == (31, 24) and shp["ve_gate.0"] == (3, om.VE_GATE_CH) and shp["smear_w"] == (24,)
    # the packed order of the input generator matches (it adds only an unused pad)
    dims = inputs.Dims.from_depth(4, 1000, n_kv_head=1, features="vsrb")
    cfg4 = om.Config.from_depth(4, 1000, n_kv_head=1, features="vsrb")
    packed = [(n, s) for n, s in inputs.packed_tensors(dims) if n != "pad"]
    assert packed == [(n, om.param_shapes(cfg4)[n]) for n in om.param_names(cfg4)]
    assert inputs.n_params(dims) % 4 == 0


def test_finite_differences_features():
    cfg = TINY_FEAT
    P = _feat_params(cfg, seed=71)
    ids = _tiny_ids(cfg, B=2, T=9, seed=72)
    out = om.forward_backward(P, ids, cfg)
    rng = np.random.default_rng(73)
    h = 1e-5
    for name in om.param_names(cfg):
        W = P[name]
        for _ in range(3):
            idx = tuple(int(rng.integers(0, s)) for s in W.shape)
            if name == "wte" or name.startswith("ve."):   # a row that is used
                idx = (int(ids[0, int(rng.integers(0, ids.shape[1] - 1))]), idx[1])
            old = W[idx]
            W[idx] = old + h
            lp = om.forward_backward(P, ids, cfg, want_grads=False)["loss"]
            W[idx] = old - h
            lm = om.forward_backward(P, ids, cfg, want_grads=False)["loss"]
            W[idx] = old
            fd = (lp - lm) / (2 * h)
            an = out["grads"][name][idx]
            assert abs(fd - an) / (abs(an) + 1e-4) < 1e-6, (name, idx, fd, an)


def test_features_against_torch_autograd():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    cfg = TINY_FEAT
    P = _feat_params(cfg, seed=81)
    ids = _tiny_ids(cfg, B=2, T=10, seed=82)
    out = om.forward_backward(P, ids, cfg)
    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in P.items()}
    B, T = ids.shape[0], ids.shape[1] - 1
    d, H, Hkv, hd, L = cfg.d_model, cfg.n_head, cfg.n_kv_head, cfg.head_dim, cfg.n_layer
    inp, tgt = torch.tensor(ids[:, :T]), torch.tensor(ids[:, 1:])
    freq = cfg.rope_base ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    rot = torch.polar(torch.ones(T, hd // 2, dtype=torch.float64),
                      torch.arange(T, dtype=torch.float64)[:, None] * freq[None, :])

    def rope_t(x):
        xc = torch.complex(x[..., : hd // 2], x[..., hd // 2:]) * rot
        return torch.cat([xc.real, xc.imag], dim=-1)

    def rms(x, n):
        return F.rms_norm(x, (n,), eps=cfg.eps)

    ii = torch.arange(T)[:, None]
    jj = torch.arange(T)[None, :]
    emb = tp["wte"][inp]                                      # [B, T, d]
    # smear: shift the embeddings one step along the sequence (zero before the first)
    shifted = F.pad(emb, (0, 0, 1, 0))[:, :T]
    gate = tp["smear_lambda"] * torch.sigmoid(emb[..., :24] @ tp["smear_w"])
    x = emb + gate.unsqueeze(-1) * shifted
    x0 = x
    for i in range(L):
        x = tp["resid_lambda"][i] * x + tp["x0_lambda"][i] * x0
        h = rms(x, d)
        q = (h @ tp[f"wq.{i}"].T).view(B, T, H, hd).transpose(1, 2)
        k = (h @ tp[f"wk.{i}"].T).view(B, T, Hkv, hd).transpose(1, 2)
        v = (h @ tp[f"wv.{i}"].T).view(B, T, Hkv, hd)
        if i % 2 == 0:
            g = 3 * torch.sigmoid(h[..., :32] @ tp[f"ve_gate.{i}"].T)      # [B, T, Hkv]
            v = v + g.unsqueeze(-1) * tp[f"ve.{i}"][inp].view(B, T, Hkv, hd)
        v = v.transpose(1, 2)
        q, k = rms(rope_t(q), hd), rms(rope_t(k), hd)
        w = cfg.layer_window(i)
        allowed = jj <= ii if w is None else (jj <= ii) & (jj >= ii - w)
        y = F.scaled_dot_product_attention(q, k.repeat_interleave(H // Hkv, dim=1),
                                           v.repeat_interleave(H // Hkv, dim=1), attn_mask=allowed)
        x = x + y.transpose(1, 2).reshape(B, T, d) @ tp[f"wo.{i}"].T
        h = rms(x, d)
        x = x + F.relu(h @ tp[f"wfc.{i}"].T).square() @ tp[f"wproj.{i}"].T
        if i == L // 2 - 1:
            x_mid = x
    x = x - tp["backout_lambda"] * x_mid
    z = rms(x, d) @ tp["lm_head"].T
    loss = F.cross_entropy(z.reshape(-1, cfg.vocab), tgt.reshape(-1))
    loss.backward()
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-12)
    for name in om.param_names(cfg):
        ref = tp[name].grad.numpy()
        assert np.abs(out["grads"][name] - ref).max() <= 1e-11 * max(1.0, np.abs(ref).max()), name


def test_features_at_neutral_values_are_the_plain_model():
    cfg = TINY_FEAT
    plain = om.Config(**{**cfg.__dict__, "value_embeds": False, "smear": False, "resid_lambdas": False,
                         "backout": False})
    P = _feat_params(cfg, seed=91)
    P["resid_lambda"][:] = 1.0
    P["x0_lambda"][:] = 0.0
    P["smear_lambda"][:] = 0.0
    P["backout_lambda"][:] = 0.0
    for i in cfg.ve_layers():
        P[f"ve.{i}"][:] = 0.0
    ids = _tiny_ids(cfg, B=2, T=9, seed=92)
    a = om.forward_backward(P, ids, cfg)
    b = om.forward_backward({n: P[n] for n in om.param_names(plain)}, ids, plain)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-13)
    for name in om.param_names(plain):
        assert np.allclose(a["grads"][name], b["grads"][name], rtol=1e-11, atol=1e-14), name


def test_features_are_causal():
    """The loss of position t does not depend on inputs after t (smear reads the
    previous token, never the next)."""
    cfg = TINY_FEAT
    P = _feat_params(cfg, seed=93)
    ids = _tiny_ids(cfg, B=1, T=9, seed=94)
    base = om.forward_backward(P, ids, cfg, want_grads=False)["row_loss"][0]
    ids2 = ids.copy()
    ids2[0, 6] = (ids2[0, 6] + 5) % cfg.vocab        # input of position 6 (target of position 5)
    alt = om.forward_backward(P, ids2, cfg, want_grads=False)["row_loss"][0]
    assert np.array_equal(base[:5], alt[:5])
    assert not np.allclose(base[6:], alt[6:])


def test_smear_leaves_the_first_position():
    cfg = om.Config(**{**TINY_FEAT.__dict__, "value_embeds": False, "resid_lambdas": False, "backout": False})
    plain = om.Config(**{**cfg.__dict__, "smear": False})
    P = _feat_params(cfg, seed=95)
    ids = _tiny_ids(cfg, B=2, T=9, seed=96)
    a = om.forward_backward(P, ids, cfg, want_grads=False)["row_loss"]
    b = om.forward_backward({n: P[n] for n in om.param_names(plain)}, ids, plain, want_grads=False)["row_loss"]
    assert np.array_equal(a[:, 0], b[:, 0])
    assert not np.allclose(a[:, 1:], b[:, 1:])


def test_first_layer_lambdas_have_equal_gradients():
    """Layer 0's input is x0 itself, so resid_lambda[0] and x0_lambda[0] act
    on the same tensor: equal gradients, and only their sum matters."""
    cfg = TINY_FEAT
    P = _feat_params(cfg, seed=97)
    ids = _tiny_ids(cfg, B=2, T=9, seed=98)
    out = om.forward_backward(P, ids, cfg)
    assert out["grads"]["resid_lambda"][0] == out["grads"]["x0_lambda"][0]
    P2 = {k: v.copy() for k, v in P.items()}
    P2["resid_lambda"][0], P2["x0_lambda"][0] = P["x0_lambda"][0], P["resid_lambda"][0]
    assert om.forward_backward(P2, ids, cfg, want_grads=False)["loss"] == pytest.approx(out["loss"], rel=1e-14)


def test_grad_abs_bounds_the_scalar_gradients():
    """grad_abs is the sum of the absolute values of the terms of each scalar
    gradient: never below the gradient's magnitude (triangle inequality), and
    additive over sequence chunks."""
    cfg = TINY_FEAT
    P = _feat_params(cfg, seed=99)
    ids = _tiny_ids(cfg, B=2, T=9, seed=100)
    out = om.forward_backward(P, ids, cfg)
    for name, a in out["grad_abs"].items():
        assert np.all(a >= np.abs(out["grads"][name]) * (1 - 1e-12)), name
        assert np.all(np.isfinite(a)), name
    # chunked processing adds the per-chunk sums
    chunked = om.forward_backward(P, ids, cfg, seq_chunk=1)
    for name, a in out["grad_abs"].items():
        assert np.allclose(chunked["grad_abs"][name], a, rtol=1e-12), name
