"""Run the HIP step and the oracle on the same seeded inputs (GPU tests)."""

import numpy as np
import torch

from gpt_transformer_step_amd import inputs
from oracle import model as om
from oracle import precision
from gpu_util import say


class StepRun:
    """Device buffers of one configuration, filled from the seeded generators."""

    def __init__(self, depth, vocab, seq_len, batch, seed_ids=inputs.SEED_IDS, seed_w=inputs.SEED_W,
                 precision_flag=0, n_kv_head=0, window=0, pattern="", features=""):
        from gpt_transformer_step_amd import binding as B
        self.B = B
        self.dims = inputs.Dims.from_depth(depth, vocab, n_kv_head, features=features)
        self.depth, self.vocab, self.T, self.batch = depth, vocab, seq_len, batch
        self.n_kv_head, self.window, self.pattern, self.features = n_kv_head, window, pattern, features
        self.shape = B.shape(depth, vocab, seq_len, batch, precision_flag, n_kv_head=n_kv_head, window=window,
                             pattern=pattern, features=features)
        self.n = B.param_count(self.shape)
        assert self.n == inputs.n_params(self.dims)
        self.master_np = inputs.master_weights(self.dims, seed_w)
        self.ids_np = inputs.token_ids(batch, seq_len, vocab, seed_ids)
        dev = torch.device("cuda:0")
        self.master = torch.from_numpy(self.master_np).to(dev)
        self.bf16 = torch.empty(self.n, dtype=torch.bfloat16, device=dev)
        B.cast_bf16(self.master, self.bf16)
        self.grad = torch.full((self.n,), float("nan"), dtype=torch.float32, device=dev)
        self.ids = torch.from_numpy(self.ids_np).to(dev)
        self.ws = torch.empty(B.workspace_size(self.shape), dtype=torch.uint8, device=dev)
        self.params = B.make_params(self.master, self.bf16, self.grad)
        self.loss = torch.zeros(1, dtype=torch.float32, device=dev)
        self.row_lse = torch.zeros(batch * seq_len, dtype=torch.float32, device=dev)

    def fwd(self, logits=None):
        self.B.step_fwd(self.shape, self.params, self.ids, self.loss, self.ws, row_lse=self.row_lse,
                        logits=logits)

    def bwd(self, accumulate=False):
        self.B.step_bwd(self.shape, self.params, self.ids, self.ws, accumulate=accumulate)

    def ws_tensor(self, which, layer=0, dtype=torch.float32):
        off, nb = self.B.workspace_tensor(self.shape, which, layer)
        return self.ws[off: off + nb].view(dtype)

    def grads(self):
        g = self.grad.cpu().numpy()
        return inputs.unpack(self.dims, g)

    def oracle_params(self):
        """bf16 values of the master weights (what the step computes with)."""
        vals = precision.round_bf16(self.master_np)
        return {k: v.astype(np.float64) for k, v in inputs.unpack(self.dims, vals).items()}

    def oracle_cfg(self):
        return om.Config.from_depth(self.depth, self.vocab, self.n_kv_head, self.window, self.pattern or "L",
                                    self.features)


def oracle_run(run, want_logits=False, dtype=np.float64, seq_chunk=None, fp8=False, bf16_operands=False):
    say(f"oracle: depth={run.depth} V={run.vocab} T={run.T} B={run.batch} bf16_operands={bf16_operands}")
    return om.forward_backward(run.oracle_params(), run.ids_np, run.oracle_cfg(), dtype=dtype,
                               want_logits=want_logits, seq_chunk=seq_chunk, fp8=fp8,
                               bf16_operands=bf16_operands)
