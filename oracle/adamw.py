"""Oracle of the AdamW update for the embedding and head matrices (numpy).

Test infrastructure only.  The optimizer passage of the pages (dev.to
"¿Cómo Entrenar Tu Propio ChatGPT por $50?", section "2. Optimizador Muon
(nanochat/optim.py)"; apidog.com/pt "Otimizador Muon") assigns AdamW to the
token embedding, the output matrix and scalar parameters, and Muon to the 2-D
block matrices.  The pages give no AdamW hyperparameters; they are inputs.

Readings taken (the textbook algorithm: Loshchilov & Hutter, "Decoupled
Weight Decay Regularization", ICLR 2019, Adam with decoupled weight decay):
  * g = grad_scale * G (grad_scale lets accumulated micro-batch gradients be
    averaged);
  * m <- beta1 m + (1 - beta1) g,  v <- beta2 v + (1 - beta2) g^2, m = v = 0
    before step 1;
  * m_hat = m / (1 - beta1^t), v_hat = v / (1 - beta2^t) for step t >= 1;
  * W <- W (1 - lr wd) - lr m_hat / (sqrt(v_hat) + eps).

Pinned by (tests/test_oracle_adamw.py): torch's CPU torch.optim.AdamW (a
library implementation of the same algorithm) over several steps; the first
step from a zero state moves every weight by lr g / (|g| + eps); weight decay
alone (g = 0) scales W by (1 - lr wd) per step.
"""

import numpy as np


def adamw_update(W, G, M, V, step, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, grad_scale=1.0,
                 dtype=np.float64):
    """One AdamW step.  W, M, V are updated in place (arrays of `dtype`);
    returns W.  step is the 1-based count of this update."""
    if step < 1:
        raise ValueError("step is 1-based")
    g = np.asarray(G, dtype=dtype) * dtype(grad_scale)
    M *= beta1
    M += (1.0 - beta1) * g
    V *= beta2
    V += (1.0 - beta2) * g * g
    m_hat = M / (1.0 - beta1 ** step)
    v_hat = V / (1.0 - beta2 ** step)
    W *= (1.0 - lr * weight_decay)
    W -= lr * m_hat / (np.sqrt(v_hat) + eps)
    return W
