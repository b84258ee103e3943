"""Oracle of the Muon update for 2-D weight matrices (numpy).

Test infrastructure only.  The optimizer passage of the pages (dev.to
"¿Cómo Entrenar Tu Propio ChatGPT por $50?", section "2. Optimizador Muon
(nanochat/optim.py)"; apidog.com/pt "Otimizador Muon"; apidog.com/de
"Muon-Optimierer") states: 2-D matrices are updated by Muon (momentum, then
orthogonalisation by a Newton-Schulz iteration with Polar-Express
coefficients, five iterations); each iteration takes a coefficient triple
(a, b, c) and computes A = X^T X, B = b A + c A A, X = a X + X B.

Readings taken:
  * momentum M <- mu M + G with M = 0 before the first step, no Nesterov term;
  * X0 = M / (||M||_F + 1e-7); the loop runs on the orientation with
    rows >= cols (X^T X is the small Gram matrix) and the result is
    transposed back;
  * the coefficient table is an input (the pages print only its first two
    triples); the update is W <- W (1 - lr wd) - lr X.

NorMuon variance reduction (normuon_scale; dev.to section "2. Optimizador
Muon", "Reducción de varianza NorMuon"; apidog.com/pt "Redução de Variância
NorMuon"): after the orthogonalisation the update is rescaled per neuron so
that no neuron's scale collapses, keeping the overall size of the update.
The pages show only the first and last lines (per-neuron mean squares, their
summed norm, the final scale = step size x norm before / norm after); the
middle is completed with the published NorMuon algorithm (Li et al., 2025,
"NorMuon: Making Muon more efficient and scalable"):
  * a neuron is a row of the [out, in] matrix (statistic over the inputs);
    axis=0 takes columns instead (the pages leave the reduced dimension a
    variable);
  * vm_i = mean of O_i^2 over the neuron's weights; V <- beta2 V + (1-beta2) vm
    with V = 0 before the first step and no bias correction;
  * step_i = 1 / (sqrt(V_i) + eps);
  * norm_before = sqrt(sum_i vm_i), norm_after = sqrt(sum_i vm_i step_i^2)
    (the same measure of O scaled by step);
  * O'_i = O_i * step_i * norm_before / max(norm_after, 1e-10).
A bias correction of V would multiply every step_i by one factor, which the
norm ratio cancels (up to eps).

Pinned by (tests/test_oracle_muon.py): for any table, the result equals
U diag(p_k(...p_1(sigma / (||G|| + eps)))) V^T computed from a float64 LAPACK
SVD (each iteration applies the odd polynomial p(s) = a s + b s^3 + c s^5 to
the singular values); the textbook quintic iterated many times converges to
the polar factor U V^T; at the first step the update does not depend on mu
or on the scale of the gradient.  NorMuon: the rescale keeps the Frobenius
norm; from V = 0 (eps -> 0) it gives every neuron the same RMS, so an update
whose neurons already share one RMS (rows of a semi-orthogonal matrix) comes
back unchanged; V after several steps equals the closed-form weighted sum
(1 - beta2) sum_s beta2^(t-s) vm_s; scaling O by c (and V by c^2) scales O'
by c; permuting neurons permutes the result; axis=0 equals axis=1 on the
transpose.
"""

import numpy as np


def newton_schulz(G, coeffs, eps=1e-7):
    """Orthogonalise G with the iteration X <- a X + X (b X^T X + c (X^T X)^2)
    for each (a, b, c) in coeffs, starting from G / (||G||_F + eps)."""
    X = np.asarray(G, dtype=np.float64)
    X = X / (np.linalg.norm(X) + eps)
    tall = X.shape[0] >= X.shape[1]
    if not tall:
        X = X.T
    for a, b, c in coeffs:
        A = X.T @ X
        Bm = b * A + c * (A @ A)
        X = a * X + X @ Bm
    return X if tall else X.T


def muon_update(W, G, M, coeffs, lr, momentum, weight_decay, eps=1e-7):
    """One Muon step for one matrix.  Returns (W_new, M_new, O) where O is the
    orthogonalised update."""
    M_new = momentum * np.asarray(M, dtype=np.float64) + np.asarray(G, dtype=np.float64)
    O = newton_schulz(M_new, coeffs, eps)
    W_new = np.asarray(W, dtype=np.float64) * (1.0 - lr * weight_decay) - lr * O
    return W_new, M_new, O


def normuon_scale(O, V, beta2=0.95, eps=1e-8, axis=1):
    """NorMuon rescale of an orthogonalised update O [rows, cols].  V holds one
    second moment per neuron (rows when axis=1, columns when axis=0) and is
    updated in place.  Returns the rescaled update."""
    O = np.asarray(O, dtype=np.float64)
    vm = np.mean(O * O, axis=axis)                 # per-neuron mean square
    norm_before = np.sqrt(np.sum(vm))
    V *= beta2
    V += (1.0 - beta2) * vm
    step = 1.0 / (np.sqrt(V) + eps)
    norm_after = np.sqrt(np.sum(vm * step * step))
    scale = step * (norm_before / max(norm_after, 1e-10))
    return O * (scale[:, None] if axis == 1 else scale[None, :])


def normuon_update(W, G, M, V, coeffs, lr, momentum, weight_decay, beta2=0.95, eps_v=1e-8, axis=1, eps=1e-7):
    """One Muon step with the NorMuon rescale between the orthogonalisation and
    the update.  V is updated in place.  Returns (W_new, M_new, O') with O' the
    rescaled update."""
    M_new = momentum * np.asarray(M, dtype=np.float64) + np.asarray(G, dtype=np.float64)
    O = normuon_scale(newton_schulz(M_new, coeffs, eps), V, beta2, eps_v, axis)
    W_new = np.asarray(W, dtype=np.float64) * (1.0 - lr * weight_decay) - lr * O
    return W_new, M_new, O


# The textbook quintic Newton-Schulz step for the matrix sign / polar factor:
# the degree-2 truncation of the binomial series of (1 - t)^(-1/2) at t = 1 - s^2
# gives p(s) = s (15 - 10 s^2 + 3 s^4) / 8 (Higham, Functions of Matrices, 2008).
NS5_QUINTIC = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)
