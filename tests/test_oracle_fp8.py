"""Pins of the software fp8 codec and of bf16 rounding (oracle side)."""

import numpy as np
import pytest

from oracle import fp8, precision


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_every_finite_code_roundtrips(fmt):
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8.decode(codes, fmt)
    fin = np.isfinite(vals)
    back = fp8.encode(vals[fin], fmt)
    # every finite code is its own image (-0.0 included)
    assert np.array_equal(back, codes[fin])


def test_format_constants():
    assert fp8.fmax("e4m3") == 448.0
    assert fp8.fmax("e5m2") == 57344.0
    assert np.isnan(fp8.decode(np.uint8(0x7F), "e4m3"))
    assert np.isinf(fp8.decode(np.uint8(0x7C), "e5m2"))
    assert fp8.decode(np.uint8(1), "e4m3") == 2.0 ** -9
    assert fp8.decode(np.uint8(1), "e5m2") == 2.0 ** -16


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_midpoints_round_to_even_and_saturate(fmt):
    table = fp8.decode(np.arange(128), fmt)
    table = table[np.isfinite(table)]
    mids = 0.5 * (table[:-1] + table[1:])
    codes = fp8.encode(mids, fmt)
    assert np.all(codes % 2 == 0)
    assert np.all(np.abs(codes.astype(int) - np.arange(len(mids))) <= 1)
    big = np.array([fp8.fmax(fmt) * 1.01, 1e30, -1e30])
    dec = fp8.decode(fp8.encode(big, fmt), fmt)
    assert np.array_equal(np.abs(dec), np.full(3, fp8.fmax(fmt)))


@pytest.mark.parametrize("fmt,tdt", [("e4m3", "float8_e4m3fn"), ("e5m2", "float8_e5m2")])
def test_against_torch_casts(fmt, tdt):
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(0)
    fm = fp8.fmax(fmt)
    x = np.concatenate([g.uniform(-fm, fm, 20000), g.standard_normal(20000) * 1e-3,
                        g.standard_normal(20000) * 10]).astype(np.float32)
    x = np.clip(x, -fm, fm)
    ours = fp8.decode(fp8.encode(x, fmt), fmt)
    ref = torch.tensor(x).to(getattr(torch, tdt)).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    # the codes themselves, including the sign of values that round to zero
    tiny = np.array([-1e-6, 1e-6, -0.0, 0.0, -fp8.decode(np.uint8(1), fmt) * 0.49], np.float32)
    codes = fp8.encode(np.concatenate([x, tiny]), fmt)
    ref_codes = torch.tensor(np.concatenate([x, tiny])).to(getattr(torch, tdt)).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref_codes)
    assert list(codes[-5:]) == [0x80, 0, 0x80, 0, 0x80]


def test_fake_quant_scale():
    g = np.random.default_rng(1)
    t = g.standard_normal((32, 16)) * 0.01
    fq = fp8.fake_quant(t, "e4m3")
    # the element of largest magnitude lands exactly on fmax / s
    i = np.unravel_index(np.argmax(np.abs(t)), t.shape)
    assert fq[i] == pytest.approx(t[i], rel=1e-6)
    assert np.abs(fq - t).max() <= np.abs(t).max() * 2 ** -4
    assert np.array_equal(fp8.fake_quant(np.zeros(4), "e5m2"), np.zeros(4))


def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(2)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.4e38, -3.4e38, 1e-40, np.inf, -np.inf], np.float32)])
    ours = precision.bf16_bits(x)
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert precision.round_bf16(np.array([1 + 2 ** -8], np.float32))[0] == 1.0
    assert precision.round_bf16(np.array([1 + 3 * 2 ** -8], np.float32))[0] == 1 + 2 ** -6
