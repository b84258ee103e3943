"""One GPT pretraining step (forward, backward, Muon) on AMD MI355X.

The compute lives in ``libgptstep.so`` (hand-written HIP kernels for gfx950
behind a C ABI, declared in ``include/gptstep.h``).  ``binding`` is a thin
ctypes layer over it.  Importing this package does not load the library (use
``from gpt_transformer_step_amd import binding``), so that ``inputs`` can be
used on machines without a GPU.
"""
