"""Pins of the storage roundings (oracle/rounding.py) on hand-derived bit
patterns, and of the bf16 rounding against torch's own conversion."""

import numpy as np
import pytest

from oracle import fp16_rne, f32_to_bf16_rne_bits, bf16_bits_to_f64

F16_CASES = [
    (1.0, 0x3C00),
    (1.0 + 2.0 ** -11, 0x3C00),                 # tie -> even (down)
    (1.0 + 3 * 2.0 ** -11, 0x3C02),             # tie -> even (up)
    (1.0 + 2.0 ** -11 + 2.0 ** -40, 0x3C01),    # direct rounding; via fp32 it would tie down
    (2.0 ** -24, 0x0001),                       # smallest subnormal
    (2.0 ** -25, 0x0000),                       # half of it: tie -> even 0
    (2.0 ** -25 + 2.0 ** -60, 0x0001),
    (3 * 2.0 ** -25, 0x0002),                   # 1.5 ulp: tie -> even 2
    (2.0 ** -14, 0x0400),                       # smallest normal
    (2.0 ** -14 - 2.0 ** -25, 0x0400),          # 1023.5 ulp: tie -> even 1024
    (2.0 ** -14 - 2.0 ** -24, 0x03FF),          # largest subnormal
    (65504.0, 0x7BFF),
    (65519.99, 0x7BFF),
    (65520.0, 0x7C00),                          # tie above max -> inf
    (-0.0, 0x8000),
    (-3.0, 0xC200),
    (0.1, 0x2E66),                              # 0.0999755859375
]


@pytest.mark.parametrize("v,bits", F16_CASES)
def test_fp16_rne_bits(v, bits):
    assert int(fp16_rne(np.array([v]))[0].view(np.uint16)) == bits


BF16_CASES = [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                  # tie -> even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),              # tie -> even up
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),
    (-2.5, 0xC020),
    (3.4028234663852886e38, 0x7F80),            # fp32 max rounds up to inf
    (3.3895313892515355e38, 0x7F7F),            # bf16 max is exact
    (1e-40, 0x0001),                            # fp32 subnormal 0x000116C2 -> 0x0001
]


@pytest.mark.parametrize("v,bits", BF16_CASES)
def test_bf16_rne_bits(v, bits):
    assert int(f32_to_bf16_rne_bits(np.array([v], np.float32))[0]) == bits


def test_bf16_matches_torch_random():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(5)
    x = np.concatenate([
        g.standard_normal(200000).astype(np.float32),
        (g.standard_normal(20000) * 1e-39).astype(np.float32),
        np.array([np.inf, -np.inf, 0.0, -0.0], np.float32),
        g.integers(0, 2 ** 32, 50000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[~np.isnan(x)]
    ours = f32_to_bf16_rne_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_nan_stays_nan():
    b = f32_to_bf16_rne_bits(np.array([np.nan], np.float32))
    assert np.isnan(bf16_bits_to_f64(b))[0]


def test_bf16_widening_exact():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    back = f32_to_bf16_rne_bits(v[fin].astype(np.float32))
    np.testing.assert_array_equal(back, bits[fin])
