"""Pins of the Muon oracle: SVD closed form, polar-factor limit, invariances,
and the coefficient triples the pages print."""

import json
import os

import numpy as np
import pytest

from oracle import muon as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


def _svd_closed_form(G, coeffs, eps=1e-7):
    """U diag(p_k(...p_1(s))) V^T with s the singular values of G/(||G||+eps)."""
    U, s, Vt = np.linalg.svd(np.asarray(G, dtype=np.float64), full_matrices=False)
    s = s / (np.linalg.norm(G) + eps)
    for a, b, c in coeffs:
        s = a * s + b * s ** 3 + c * s ** 5
    return (U * s) @ Vt


@pytest.mark.parametrize("shape", [(12, 5), (5, 12), (9, 9), (64, 16)])
def test_ns_equals_svd_closed_form(shape):
    g = np.random.default_rng(1)
    G = g.standard_normal(shape)
    tables = [
        [om.NS5_QUINTIC] * 5,
        [tuple(g.uniform(-2, 3, size=3)) for _ in range(3)],
        json.load(open(GOLDEN))["polar_express_printed_triples"],
    ]
    for coeffs in tables:
        got = om.newton_schulz(G, coeffs)
        ref = _svd_closed_form(G, coeffs)
        assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_ns5_converges_to_polar_factor():
    g = np.random.default_rng(2)
    for shape in [(30, 10), (10, 30), (16, 16)]:
        G = g.standard_normal(shape)
        U, _, Vt = np.linalg.svd(G, full_matrices=False)
        X = om.newton_schulz(G, [om.NS5_QUINTIC] * 60)
        assert np.abs(X - U @ Vt).max() < 1e-9


def test_first_step_invariances():
    g = np.random.default_rng(3)
    W = g.standard_normal((8, 20))
    G = g.standard_normal((8, 20))
    M0 = np.zeros_like(G)
    coeffs = [om.NS5_QUINTIC] * 5
    _, _, O1 = om.muon_update(W, G, M0, coeffs, 0.02, 0.95, 0.0)
    _, _, O2 = om.muon_update(W, G, M0, coeffs, 0.02, 0.5, 0.0)
    _, _, O3 = om.muon_update(W, 7.0 * G, M0, coeffs, 0.02, 0.95, 0.0)
    assert np.abs(O1 - O2).max() < 1e-15
    assert np.abs(O1 - O3).max() < 1e-6  # only the eps in the norm differs


def test_update_rule():
    g = np.random.default_rng(4)
    W = g.standard_normal((6, 4))
    G = g.standard_normal((6, 4))
    M = g.standard_normal((6, 4))
    coeffs = [om.NS5_QUINTIC] * 2
    Wn, Mn, O = om.muon_update(W, G, M, coeffs, 0.1, 0.9, 0.5)
    assert np.allclose(Mn, 0.9 * M + G)
    assert np.allclose(Wn, W * (1 - 0.05) - 0.1 * O)


def test_printed_triples_fixture():
    data = json.load(open(GOLDEN))
    t = data["polar_express_printed_triples"]
    assert t == [[8.156, -22.483, 15.879], [4.043, -2.809, 0.5]]
    assert data["ns_steps"] == 5
    # each printed polynomial is odd with slope a at 0 and maps (0, 1] into
    # (0, 2): singular values grow towards 1 and none changes sign
    s = np.linspace(1e-3, 1, 20001)
    for a, b, c in t:
        p = a * s + b * s ** 3 + c * s ** 5
        assert p.min() > 0 and p.max() < 2
        assert np.all(p[s < 0.1] > s[s < 0.1])


# ---------------------------------------------------------------------------
# NorMuon rescale
# ---------------------------------------------------------------------------

def _uneven(g, rows, cols):
    """A matrix whose rows have very different scales."""
    return g.standard_normal((rows, cols)) * np.exp(g.uniform(-3, 3, (rows, 1)))


@pytest.mark.parametrize("axis", [1, 0])
def test_normuon_keeps_frobenius_norm(axis):
    g = np.random.default_rng(10)
    V = np.abs(g.standard_normal(24 if axis == 1 else 40)) * 0.3
    for _ in range(3):
        O = _uneven(g, 24, 40)
        out = om.normuon_scale(O, V, 0.9, 1e-8, axis)
        assert np.isclose(np.linalg.norm(out), np.linalg.norm(O), rtol=1e-12)


def test_normuon_first_step_equalises_neurons():
    g = np.random.default_rng(11)
    O = _uneven(g, 30, 17)
    V = np.zeros(30)
    out = om.normuon_scale(O, V, 0.95, 0.0)
    rms = np.sqrt(np.mean(out * out, axis=1))
    # every neuron gets the RMS of the whole update
    assert np.allclose(rms, np.linalg.norm(O) / np.sqrt(O.size), rtol=1e-12)


def test_normuon_leaves_semi_orthogonal_rows_unchanged():
    g = np.random.default_rng(12)
    Q, _ = np.linalg.qr(g.standard_normal((48, 16)))
    O = Q.T                                            # 16 x 48, orthonormal rows
    out = om.normuon_scale(O, np.zeros(16), 0.95, 1e-8)
    assert np.allclose(out, O, rtol=1e-7, atol=1e-12)
    # and the Newton-Schulz output of a wide matrix is nearly such a matrix
    X = om.newton_schulz(g.standard_normal((16, 48)), [om.NS5_QUINTIC] * 30)
    assert np.allclose(om.normuon_scale(X, np.zeros(16), 0.95, 1e-8), X, atol=1e-9)


def test_normuon_second_moment_closed_form():
    """After t steps V is the weighted sum (1 - b) sum_s b^(t-s) vm_s."""
    g = np.random.default_rng(13)
    beta2, rows, cols, t = 0.8, 9, 14, 5
    V = np.zeros(rows)
    hist = []
    for _ in range(t):
        O = _uneven(g, rows, cols)
        hist.append(np.mean(O * O, axis=1))
        om.normuon_scale(O, V, beta2, 1e-8)
    ref = (1 - beta2) * sum(beta2 ** (t - 1 - s) * vm for s, vm in enumerate(hist))
    assert np.allclose(V, ref, rtol=1e-13)


def test_normuon_beta2_zero_forgets_history():
    g = np.random.default_rng(14)
    V = np.abs(g.standard_normal(12)) * 5.0
    O = _uneven(g, 12, 20)
    out = om.normuon_scale(O, V, 0.0, 0.0)
    rms = np.sqrt(np.mean(out * out, axis=1))
    assert np.allclose(rms, rms[0], rtol=1e-12)


def test_normuon_homogeneous_and_equivariant():
    g = np.random.default_rng(15)
    O = _uneven(g, 10, 6)
    V0 = np.abs(g.standard_normal(10))
    base = om.normuon_scale(O, V0.copy(), 0.9, 0.0)
    c = 3.7
    assert np.allclose(om.normuon_scale(c * O, c * c * V0.copy(), 0.9, 0.0), c * base, rtol=1e-12)
    perm = g.permutation(10)
    assert np.allclose(om.normuon_scale(O[perm], V0[perm].copy(), 0.9, 0.0), base[perm], rtol=1e-12)
    # statistic over columns = statistic over rows of the transpose
    Vc = np.abs(g.standard_normal(6))
    assert np.allclose(om.normuon_scale(O, Vc.copy(), 0.9, 1e-8, axis=0),
                       om.normuon_scale(O.T, Vc.copy(), 0.9, 1e-8, axis=1).T, rtol=1e-14)


def test_normuon_update_composes():
    g = np.random.default_rng(16)
    W, G, M = (g.standard_normal((20, 12)) for _ in range(3))
    V = np.zeros(20)
    lr, mu, wd = 0.02, 0.9, 0.1
    Wn, Mn, O = om.normuon_update(W, G, M, V, [om.NS5_QUINTIC] * 5, lr, mu, wd, beta2=0.95)
    assert np.allclose(Mn, mu * M + G)
    assert np.allclose(Wn, W * (1 - lr * wd) - lr * O)
    # O is the rescaled orthogonalisation: same Frobenius norm as the plain one
    plain = om.newton_schulz(Mn, [om.NS5_QUINTIC] * 5)
    assert np.isclose(np.linalg.norm(O), np.linalg.norm(plain), rtol=1e-12)
    # and from V = 0 each of its rows has the same RMS (eps = 1e-8 is negligible here)
    rms = np.sqrt(np.mean(O * O, axis=1))
    assert np.allclose(rms, rms.mean(), rtol=1e-6)
