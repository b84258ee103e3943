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

Pinned by (tests/test_oracle_muon.py): for any table, the result equals
U diag(p_k(...p_1(sigma / (||G|| + eps)))) V^T computed from a float64 LAPACK
SVD (each iteration applies the odd polynomial p(s) = a s + b s^3 + c s^5 to
the singular values); the textbook quintic iterated many times converges to
the polar factor U V^T; at the first step the update does not depend on mu
or on the scale of the gradient.
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


# The textbook quintic Newton-Schulz step for the matrix sign / polar factor:
# the degree-2 truncation of the binomial series of (1 - t)^(-1/2) at t = 1 - s^2
# gives p(s) = s (15 - 10 s^2 + 3 s^4) / 8 (Higham, Functions of Matrices, 2008).
NS5_QUINTIC = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)
