"""CPU oracle for one GPT pretraining step (test infrastructure only).

This package is the plain, slow, obviously-correct definition that the HIP
library is checked against.  It is test infrastructure: only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it, and nothing in the product path (``gpt_transformer_step_amd``) imports it
or shares code with it.

Sources (the pages this implements; all describe nanochat):
  * dev.to, "¿Cómo Entrenar Tu Propio ChatGPT por $50?" -- section
    "Cómo Funciona nanochat": "1. Modelo GPT (nanochat/gpt.py)" (RoPE, QK norm,
    untied embeddings, ReLU^2 MLP, Flash Attention), "2. Optimizador Muon
    (nanochat/optim.py)" (Polar-Express Newton-Schulz loop), "3. Gestión de
    Precisión (nanochat/common.py)" (fp32 master, bf16 compute, fp8 option).
  * apidog.com/pt, "train-your-own-chatgpt" -- the Portuguese version of the
    same sections ("Gerenciamento de Precisão": per-tensor scaled Float8Linear).
  * apidog.com/de -- "Präzisionsverwaltung" (tensorwise fp8 scaling).
  * news.hamidun.com -- habrGPT, fp8 versus bf16.

Modules:
  model   -- forward/backward of the decoder-only transformer step.
  muon    -- Muon momentum, Newton-Schulz orthogonalisation, apply.
  adamw   -- AdamW (decoupled weight decay) for the embedding and head.
  fp8     -- software OCP E4M3 / E5M2 codec and per-tensor fake quantisation.
  precision -- round-to-nearest-even fp32 -> bf16.

Parity status of every function is recorded in its docstring; every function
here is pinned by a ``-m "not gpu"`` test (finite differences, brute force,
closed forms, library routines).  No function is "parity unpinned" except the
whole-model result at the full configuration sizes, for which the pages print
no worked example (its parts are pinned individually).
"""

from . import precision, model, muon, fp8, adamw  # noqa: F401
