"""The block sketch used by the full-size expected values
(tests/golden/make_golden.py) measures what it claims: it is linear, every
element of a tensor enters it, and the sketch-estimated relative distance of
two tensors matches the true one to within a few of its stated standard
deviations sqrt(1 / (2 n))."""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import make_golden as mg  # noqa: E402


def test_sketch_is_linear_and_sees_every_element():
    g = np.random.default_rng(3)
    a = g.standard_normal((300, 520))
    b = g.standard_normal((300, 520))
    assert np.allclose(mg.sketch("t", 2 * a - b), 2 * mg.sketch("t", a) - mg.sketch("t", b))
    # a single changed element (also in the ragged last block) moves every
    # projection of its block by +-delta
    for (i, j) in [(0, 0), (299, 519), (130, 257)]:
        e = np.zeros((300, 520))
        e[i, j] = 1.0
        s = mg.sketch("t", e).reshape(mg.SKETCH_PROJ, 2, 3)
        blk = s[:, i // 256, j // 256]
        assert np.array_equal(np.abs(blk), np.ones(mg.SKETCH_PROJ))
        assert np.count_nonzero(s) == mg.SKETCH_PROJ


def test_sketch_distance_estimates_the_true_distance():
    g = np.random.default_rng(4)
    for shape, scale in [((768, 768), 1e-2), ((1280, 5120), 3e-2), ((1664, 1664), 1e-1)]:
        ref = g.standard_normal(shape)
        # a structured difference: most of it in a few rows and one block
        err = g.standard_normal(shape) * scale
        err[:64] *= 5.0
        err[256:512, 512:768] *= 3.0
        got = ref + err
        true = np.linalg.norm(err) / np.linalg.norm(ref)
        est = np.linalg.norm(mg.sketch("w", got) - mg.sketch("w", ref)) / np.linalg.norm(mg.sketch("w", ref))
        n = mg.sketch("w", ref).size
        assert abs(est / true - 1.0) <= 5 * mg.sketch_noise(n), (shape, est, true)
