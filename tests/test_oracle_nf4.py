"""Pins of the NF4 levels and quantizer (oracle/nf4.py).

The levels are pinned through the normal CDF (scipy's ``norm.cdf``), the
inverse of the quantile function used to build them; the quantizer through a
brute-force nearest-level search. The outermost probability delta itself is
parity unpinned: the pages print no NF4 level, so these tests take delta from
the oracle and pin only the construction around it.
"""

import numpy as np
from scipy.stats import norm

from oracle import nf4_levels, quantize_nf4, pack_nf4, unpack_nf4, dequant_nf4
from oracle.nf4 import NF4_DELTA
from bit_weight_quantized_qw_amd import inputs


def test_levels_shape_and_endpoints():
    L = nf4_levels()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert np.all(np.diff(L) > 0)
    assert L[0] == -1.0 and L[15] == 1.0 and L[7] == 0.0
    assert np.sum(L < 0) == 7 and np.sum(L > 0) == 8


def test_levels_are_normal_quantiles_at_even_probabilities():
    L = nf4_levels().astype(np.float64)
    top = norm.ppf(NF4_DELTA)
    # positive side: Phi(L * top) walks from 1/2 to delta in 8 equal steps
    p_pos = norm.cdf(L[8:] * top)
    steps = (NF4_DELTA - 0.5) / 8
    np.testing.assert_allclose(p_pos, 0.5 + steps * np.arange(1, 9), atol=1e-7)
    # negative side: Phi(-L * top) walks from 1/2 to delta in 7 equal steps
    p_neg = norm.cdf(-L[:7] * top)
    steps = (NF4_DELTA - 0.5) / 7
    np.testing.assert_allclose(np.sort(p_neg), 0.5 + steps * np.arange(1, 8), atol=1e-7)


def test_quantize_is_nearest_level():
    W = inputs.weight(64, 4096, workload=21)
    q, a = quantize_nf4(W)
    L = nf4_levels().astype(np.float64)
    v = (W.reshape(64, 64, 64).astype(np.float64) / a.astype(np.float64)[..., None]).reshape(64, 4096)
    brute = np.argmin(np.abs(v[..., None] - L[None, None, :]), axis=-1)
    np.testing.assert_array_equal(q, brute)
    np.testing.assert_array_equal(a, np.abs(W.reshape(64, 64, 64)).max(axis=-1))


def test_block_extremes_hit_end_levels():
    W = inputs.weight(16, 256, workload=22)
    q, a = quantize_nf4(W)
    b = W.reshape(16, 4, 64)
    am = np.argmax(np.abs(b), axis=-1)
    for n in range(16):
        for j in range(4):
            k = j * 64 + am[n, j]
            assert q[n, k] == (15 if W[n, k] > 0 else 0)


def test_zero_block():
    W = np.zeros((2, 128), np.float32)
    W[1, 64:] = inputs.weight(1, 64, workload=23)
    q, a = quantize_nf4(W)
    assert np.all(q[0] == 7) and np.all(q[1, :64] == 7)
    assert a[0, 0] == 0 and a[0, 1] == 0 and a[1, 0] == 0 and a[1, 1] > 0
    np.testing.assert_array_equal(dequant_nf4(q, a)[0], 0.0)


def test_midpoint_ties_go_low():
    L = nf4_levels().astype(np.float64)
    mids = 0.5 * (L[:-1] + L[1:])
    # with absmax 1 (a level-15 weight present) an exact midpoint goes low
    for j, m in enumerate(mids):
        if float(np.float32(m)) != m:
            continue
        w = np.zeros((1, 64), np.float32)
        w[0, 0] = 1.0
        w[0, 1] = np.float32(m)
        q, _ = quantize_nf4(w)
        assert q[0, 1] == j


def test_pack_nibbles():
    q = np.array([[3, 12, 15, 0]], np.uint8)
    np.testing.assert_array_equal(pack_nf4(q), [[0xC3, 0x0F]])
    b = np.arange(256, dtype=np.uint8)[None, :]
    np.testing.assert_array_equal(pack_nf4(unpack_nf4(b)), b)


def test_dequant_error_bounded_by_half_gap():
    W = inputs.weight(8, 512, workload=24)
    q, a = quantize_nf4(W)
    L = nf4_levels().astype(np.float64)
    err = np.abs(dequant_nf4(q, a) - W)
    gap = np.max(np.diff(L)) / 2
    bound = np.repeat(a.astype(np.float64), 64, axis=1) * gap
    assert np.all(err <= bound * (1 + 1e-12))
