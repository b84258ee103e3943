"""Software OCP 8-bit floating point codec and per-tensor fake quantisation.

Test infrastructure only.  The precision passage of the pages (apidog.com/pt
"Gerenciamento de Precisão"; apidog.com/de "Präzisionsverwaltung"; dev.to
"3. Gestión de Precisión") turns most linear layers into fp8 layers with one
scale per tensor; the habrGPT news page (news.hamidun.com, "Fp8 frente a
bf16") compares that format with bf16.  Readings:
  * formats are the OCP ones: E4M3 (bias 7, no infinities, largest finite 448)
    for activations and weights, E5M2 (bias 15, largest finite 57344) for
    output gradients;
  * scale s = fmax / amax(|t|) of the current tensor in fp32, not rounded to a
    power of two; amax == 0 gives s = 1;
  * quantise = saturate |t * s| to fmax, then round to the nearest
    representable value, ties to the even code; dequantise = decode / s.

Pinned by (tests/test_oracle_fp8.py): every finite code decodes and re-encodes
to itself; midpoints go to the even neighbour; values past fmax saturate;
in-range values agree with torch's CPU float8_e4m3fn / float8_e5m2 casts.
"""

import numpy as np

FORMATS = {
    # name: (exponent bits, mantissa bits, bias, has_inf)
    "e4m3": (4, 3, 7, False),
    "e5m2": (5, 2, 15, True),
}


def decode(code, fmt):
    """uint8 codes -> float64 values (NaN for the NaN codes, +-inf for E5M2's
    infinity codes)."""
    eb, mb, bias, has_inf = FORMATS[fmt]
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> mb) & ((1 << eb) - 1)
    m = c & ((1 << mb) - 1)
    emax = (1 << eb) - 1
    sub = m * 2.0 ** (1 - bias - mb)
    nrm = (1.0 + m / 2.0 ** mb) * 2.0 ** (e - bias)
    v = np.where(e == 0, sub, nrm) * sign
    if has_inf:
        v = np.where(e == emax, np.where(m == 0, sign * np.inf, np.nan), v)
    else:
        v = np.where((e == emax) & (m == (1 << mb) - 1), np.nan, v)
    return v


def _positive_table(fmt):
    """Sorted non-negative finite values; index == code for these codes."""
    vals = decode(np.arange(128), fmt)
    n = int(np.argmax(~np.isfinite(vals))) if not np.all(np.isfinite(vals)) else 128
    return vals[:n]


def fmax(fmt):
    return float(_positive_table(fmt)[-1])


def encode(x, fmt):
    """float array -> uint8 codes: saturate to +-fmax, round to nearest, ties to
    the even code."""
    table = _positive_table(fmt)
    x = np.asarray(x, dtype=np.float64)
    ax = np.minimum(np.abs(x), table[-1])
    hi = np.clip(np.searchsorted(table, ax, side="left"), 0, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = ax - table[lo]
    dhi = table[hi] - ax
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    # the sign bit is kept, also when the magnitude rounds to zero (IEEE-754
    # rounding gives -0 for a negative value below half the smallest step)
    return (idx | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def tensor_scale(t, fmt):
    """fmax / amax(|t|) in fp32 (1 when the tensor is all zero)."""
    amax = np.float32(np.max(np.abs(t))) if t.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(np.float32(fmax(fmt)) / amax)


def fake_quant(t, fmt):
    """Quantise-dequantise with one fp32 scale for the whole tensor:
    decode(encode(t * s)) / s.  The product t * s is formed in fp32."""
    s = tensor_scale(t, fmt)
    scaled = (np.asarray(t, dtype=np.float32) * s).astype(np.float64)
    return decode(encode(scaled, fmt), fmt) / np.float64(s)
