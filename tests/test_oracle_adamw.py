"""Pins of the AdamW oracle (oracle/adamw.py) against things other than itself."""

import numpy as np
import pytest

from oracle import adamw


def test_matches_torch_adamw_over_steps():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(0)
    W0 = g.standard_normal((37, 11))
    grads = [g.standard_normal((37, 11)) * s for s in (1.0, 0.3, 2.0, 0.01)]
    lr, b1, b2, eps, wd = 3e-3, 0.8, 0.95, 1e-8, 0.1
    p = torch.nn.Parameter(torch.tensor(W0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    W, M, V = W0.copy(), np.zeros_like(W0), np.zeros_like(W0)
    for t, G in enumerate(grads, start=1):
        p.grad = torch.tensor(G, dtype=torch.float64)
        opt.step()
        adamw.adamw_update(W, G, M, V, t, lr, b1, b2, eps, wd)
        assert np.allclose(W, p.detach().numpy(), rtol=1e-12, atol=1e-14)


def test_first_step_moves_by_scaled_sign():
    g = np.random.default_rng(1)
    W0 = g.standard_normal(1000)
    G = g.standard_normal(1000)
    W, M, V = W0.copy(), np.zeros(1000), np.zeros(1000)
    lr, eps = 0.01, 1e-8
    adamw.adamw_update(W, G, M, V, 1, lr, 0.9, 0.999, eps, 0.0)
    # bias correction makes m_hat = g and v_hat = g^2 after one step
    assert np.allclose(W0 - W, lr * G / (np.abs(G) + eps), rtol=1e-12)


def test_decoupled_weight_decay_alone():
    W0 = np.linspace(-2, 2, 9)
    W, M, V = W0.copy(), np.zeros(9), np.zeros(9)
    for t in range(1, 4):
        adamw.adamw_update(W, np.zeros(9), M, V, t, 0.1, 0.9, 0.95, 1e-8, 0.5)
    assert np.allclose(W, W0 * (1 - 0.05) ** 3, rtol=1e-14)


def test_grad_scale_equals_prescaled_gradient():
    g = np.random.default_rng(2)
    W0, G = g.standard_normal(50), g.standard_normal(50)
    a = [W0.copy(), np.zeros(50), np.zeros(50)]
    b = [W0.copy(), np.zeros(50), np.zeros(50)]
    for t in (1, 2):
        adamw.adamw_update(a[0], G, a[1], a[2], t, 1e-2, 0.9, 0.95, 1e-6, 0.0, grad_scale=0.25)
        adamw.adamw_update(b[0], 0.25 * G, b[1], b[2], t, 1e-2, 0.9, 0.95, 1e-6, 0.0)
    assert np.array_equal(a[0], b[0])
