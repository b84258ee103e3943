"""Round-to-nearest-even float32 -> bfloat16, done on the bit pattern.

The precision passage of the pages (dev.to "¿Cómo Entrenar Tu Propio ChatGPT
por $50?", section "3. Gestión de Precisión"; apidog.com/pt "Gerenciamento de
Precisão") keeps fp32 master weights and casts them to the bf16 compute dtype
for the matmuls.  The oracle therefore computes on the bf16-rounded values of
the master weights.

Pinned by: exhaustive comparison with torch's CPU ``.to(torch.bfloat16)`` on
special values and random values, and the property that every output is exactly
representable in bf16 and lies at distance <= half an ulp from the input.
"""

import numpy as np


def bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest, ties to even.

    NaN inputs map to a quiet NaN; overflow past the largest finite bf16
    rounds to infinity (IEEE behaviour)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # u + 0x7FFF + lsb stays below 2^32 for every non-NaN pattern (the largest,
    # -inf = 0xFF800000, gains at most 0x8000); NaNs are patched below
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bits_to_f32(b):
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x):
    """Value of x after rounding to bf16, returned as float32."""
    return bits_to_f32(bf16_bits(x))
