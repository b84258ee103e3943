"""Helpers shared by the GPU tests (device transfers and error metrics)."""

import numpy as np
import torch

from oracle import precision


def dev():
    return torch.device("cuda:0")


def to_dev_bf16(x):
    """float array -> device bf16 tensor with round-to-nearest-even."""
    bits = precision.bf16_bits(np.asarray(x, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).to(dev()).view(torch.bfloat16)


def bf16_values(x):
    """The float64 values a bf16 copy of x holds."""
    return precision.round_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)


def from_dev(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def cosine(got, ref):
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    den = np.linalg.norm(got) * np.linalg.norm(ref)
    return float(np.dot(got, ref) / den) if den > 0 else 1.0


def say(*a):
    print(*a, flush=True)
