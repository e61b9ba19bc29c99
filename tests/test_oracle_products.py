"""Pins of the reference products (oracle/products.py).

No page prints a worked product, so these are special cases: brute-force
double loops that decode straight from the packed bytes (sharing no code
with the vectorized unpack/dequant), one-hot inputs, independent batch
rows, and exact rational rounding for the bf16 weights the prefill uses.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import (quantize_2bit, pack_2bit, quantize_nf4, pack_nf4,
                    gemv_2bit_ref, gemv_nf4_ref, dequant_2bit, nf4_levels,
                    prefill_weight_bf16_2bit, prefill_weight_bf16_nf4,
                    gemm_prefill_ref, bf16_bits_to_f64)
from oracle.products import _fl32_of_exact_sum
from bit_weight_quantized_qw_amd import inputs

C = [Fraction(float(np.float32(v))) for v in (-1.52, -0.45, 0.45, 1.52)]


def _brute_gemv_2bit(x16, packed, S, Z, idx, W_O):
    B, K = x16.shape
    N = packed.shape[0]
    out = np.zeros((B, N))
    idx_l = list(int(i) for i in idx)
    for b in range(B):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                xv = Fraction(float(x16[b, k]))
                if k in idx_l:
                    acc += xv * Fraction(float(W_O[n, idx_l.index(k)]))
                    continue
                code = (int(packed[n, k // 4]) >> (2 * (k % 4))) & 3
                g = k // 32
                acc += xv * (Fraction(float(S[n, g])) * C[code] + Fraction(float(Z[n, g])))
            out[b, n] = float(acc)
    return out


def test_gemv_2bit_brute_force_tiny():
    W = inputs.weight(4, 64, workload=41)
    x = inputs.act_f16(2, 64, workload=41)
    idx = np.array([3, 40], np.int32)
    r = quantize_2bit(W, idx)
    packed = pack_2bit(r["q"])
    y = gemv_2bit_ref(x, r["q"], r["S"], r["Z"], idx, r["W_O"])
    yb = _brute_gemv_2bit(x, packed, r["S"], r["Z"], idx, r["W_O"])
    np.testing.assert_allclose(y, yb, rtol=1e-13, atol=1e-15)


def test_gemv_nf4_brute_force_tiny():
    W = inputs.weight(3, 128, workload=42)
    x = inputs.act_f16(1, 128, workload=42)
    q, a = quantize_nf4(W)
    packed = pack_nf4(q)
    L = [Fraction(float(v)) for v in nf4_levels()]
    y = gemv_nf4_ref(x, q, a)
    for n in range(3):
        acc = Fraction(0)
        for k in range(128):
            nib = (int(packed[n, k // 2]) >> (4 * (k % 2))) & 15
            acc += Fraction(float(x[0, k])) * Fraction(float(a[n, k // 64])) * L[nib]
        assert abs(float(acc) - y[0, n]) <= 1e-13 * max(1.0, abs(float(acc)))


def test_gemv_one_hot_reads_columns():
    W = inputs.weight(16, 128, workload=43)
    idx = np.array([7, 100], np.int32)
    r = quantize_2bit(W, idx)
    Wh = dequant_2bit(r["q"], r["S"], r["Z"])
    for k in (0, 7, 31, 32, 100, 127):
        x = np.zeros((1, 128), np.float16)
        x[0, k] = 1
        y = gemv_2bit_ref(x, r["q"], r["S"], r["Z"], idx, r["W_O"])[0]
        if k in idx:
            np.testing.assert_array_equal(y, r["W_O"][:, list(idx).index(k)].astype(np.float64))
        else:
            np.testing.assert_array_equal(y, Wh[:, k])


def test_gemv_batch_rows_are_independent():
    W = inputs.weight(32, 256, workload=44)
    x = inputs.act_f16(5, 256, workload=44)
    r = quantize_2bit(W)
    y = gemv_2bit_ref(x, r["q"], r["S"], r["Z"])
    for b in range(5):
        # BLAS may sum a single row in another order: equal to fp64 rounding
        np.testing.assert_allclose(y[b], gemv_2bit_ref(x[b:b + 1], r["q"], r["S"], r["Z"])[0],
                                   rtol=1e-12, atol=1e-14)


def test_gemv_no_outliers_equals_empty_outliers():
    W = inputs.weight(8, 64, workload=45)
    x = inputs.act_f16(1, 64, workload=45)
    r = quantize_2bit(W)
    a = gemv_2bit_ref(x, r["q"], r["S"], r["Z"])
    b = gemv_2bit_ref(x, r["q"], r["S"], r["Z"], np.zeros(0, np.int32), np.zeros((8, 0), np.float16))
    np.testing.assert_array_equal(a, b)


def _exact_f32(fr):
    """Nearest fp32 to the rational fr, ties to even, by exact comparison."""
    f = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        key = (d, int(np.array(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def _exact_bf16_bits(f32):
    fr = Fraction(float(f32))
    b = int(np.array(f32, np.float32).view(np.uint32))
    lo = (b >> 16) << 16
    cands = [np.array(lo, np.uint32).view(np.float32), np.array(lo + 0x10000, np.uint32).view(np.float32)]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - fr)
        key = (d, (int(np.array(c).view(np.uint32)) >> 16) & 1)
        if best is None or key < best[0]:
            best = (key, int(np.array(c).view(np.uint32)) >> 16)
    return best[1]


def test_prefill_weight_2bit_exact_rounding_tiny():
    W = inputs.weight(4, 64, workload=46)
    r = quantize_2bit(W)
    bits = prefill_weight_bf16_2bit(r["q"], r["S"], r["Z"])
    for n in range(4):
        for k in range(64):
            g = k // 32
            exact = Fraction(float(r["S"][n, g])) * C[r["q"][n, k]] + Fraction(float(r["Z"][n, g]))
            assert bits[n, k] == _exact_bf16_bits(_exact_f32(exact))


def test_prefill_weight_nf4_exact_rounding_tiny():
    W = inputs.weight(2, 128, workload=47)
    q, a = quantize_nf4(W)
    bits = prefill_weight_bf16_nf4(q, a)
    L = nf4_levels()
    for n in range(2):
        for k in range(128):
            exact = Fraction(float(a[n, k // 64])) * Fraction(float(L[q[n, k]]))
            assert bits[n, k] == _exact_bf16_bits(_exact_f32(exact))


def test_single_rounding_on_fp32_midpoint():
    # z sits exactly on the fp32 midpoint between 1 and 1 + 2^-23; a tiny p
    # is lost in the fp64 sum, but the exact sum is above the midpoint.
    z = np.array([1.0 + 2.0 ** -24, 1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24])
    p = np.array([2.0 ** -80, -2.0 ** -80, 0.0])
    out = _fl32_of_exact_sum(p, z)
    assert out[0] == np.float32(1.0 + 2.0 ** -23)
    assert out[1] == np.float32(1.0)
    assert out[2] == np.float32(1.0 + 2.0 ** -22)    # plain tie -> even


def test_gemm_prefill_ref_against_loops():
    X = inputs.act_bf16_bits(3, 64, workload=48)
    W = inputs.weight(5, 64, workload=48)
    r = quantize_2bit(W)
    Wb = prefill_weight_bf16_2bit(r["q"], r["S"], r["Z"])
    Y = gemm_prefill_ref(X, Wb)
    Xf = bf16_bits_to_f64(X)
    Wf = bf16_bits_to_f64(Wb)
    for m in range(3):
        for n in range(5):
            acc = sum(Fraction(Xf[m, k]) * Fraction(Wf[n, k]) for k in range(64))
            assert abs(float(acc) - Y[m, n]) <= 1e-13 * max(1.0, abs(float(acc)))


def test_prefill_anchor_columns_substituted():
    W = inputs.weight(4, 64, workload=49)
    idx = np.array([2, 33], np.int32)
    r = quantize_2bit(W, idx)
    Wb = prefill_weight_bf16_2bit(r["q"], r["S"], r["Z"], idx, r["W_O"])
    ref = oracle.f32_to_bf16_rne_bits(r["W_O"].astype(np.float32))
    np.testing.assert_array_equal(Wb[:, idx], ref)
