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
