"""Pins of the v3.2 INT4 permutation format in the oracle (oracle/int4perm.py).

The page ("Comparative Analysis" and "Method Comparison Table" of the OTF-LLM
page) fixes the shape of the format -- two 4-bit codes per byte, a uniform
symmetric grid with zero-point 0, a static channel permutation, the top 1%
channels in FP16 -- but prints no example. Pinned here against what follows
from those statements and the readings: an independent sort for the
permutation and the 2-bit anchor selection for its head, a brute-force
nearest-level search over the 15 levels with exact rationals, constructed
groups that must be recovered exactly, sign symmetry, nibble layout by
hand-written bytes, products by a double loop over the packed bytes and by
un-permuting the weights instead of permuting x, and torch's bf16 cast for
the prefill weights.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import (int4_permutation, permute_cols, quantize_int4, pack_int4, unpack_int4,
                    dequant_int4, gemv_int4_ref, prefill_weight_bf16_int4)
from bit_weight_quantized_qw_amd import inputs


def _fp16_ulp(v):
    v = np.float16(v)
    return float(np.nextafter(v, np.float16(np.inf)) - v)


def test_permutation_orders_by_score_with_ties_to_lower_channel():
    W = inputs.weight(48, 256, workload=70)
    Xp = inputs.profile(32, 256, workload=70)
    # force exact ties: duplicate two columns of W and of the profile
    W[:, 10] = W[:, 3]
    Xp[:, 10] = Xp[:, 3]
    W[:, 200] = W[:, 101]
    Xp[:, 200] = Xp[:, 101]
    perm = int4_permutation(W, Xp)
    assert sorted(perm.tolist()) == list(range(256))
    s = oracle.channel_scores(W, Xp)
    # an independent stable sort: lexsort by (channel, -score)
    want = np.lexsort((np.arange(256), -s))
    np.testing.assert_array_equal(perm, want)
    pos = {int(c): j for j, c in enumerate(perm)}
    assert pos[3] < pos[10] and pos[101] < pos[200]
    assert np.all(np.diff(s[perm]) <= 0)


@pytest.mark.parametrize("K", [5120, 1024])
def test_permutation_head_is_the_outlier_selection(K):
    """The first floor(0.01 K) channels are the set the 2-bit anchor
    selection picks at 1% (written separately, with its own pins)."""
    W = inputs.weight(64, K, workload=71)
    Xp = inputs.profile(64, K, workload=71)
    perm = int4_permutation(W, Xp)
    n = oracle.outlier_count(K, oracle.ANCHOR_FRAC_INT4)
    assert n == K // 100
    np.testing.assert_array_equal(np.sort(perm[:n]), oracle.select_outliers(W, Xp, 0.01))


def test_quantize_is_the_nearest_level_exactly():
    """Every non-anchor weight takes the nearest of the 15 levels s*q
    (q = -7..7) under exact rational arithmetic; exact ties go to even q."""
    W = inputs.weight(6, 128, workload=72)
    perm = np.random.default_rng(72).permutation(128).astype(np.int32)
    r = quantize_int4(W, perm, 3)
    Wp = permute_cols(W, perm)
    for n in range(6):
        for j in range(3, 128):
            s = Fraction(float(r["s"][n, j // 32]))
            w = Fraction(float(Wp[n, j]))
            q = int(r["q"][n, j])
            dist = [abs(w - s * k) for k in range(-7, 8)]
            best = min(dist)
            cands = [k for k in range(-7, 8) if dist[k + 7] == best]
            want = cands[0] if len(cands) == 1 else [k for k in cands if k % 2 == 0][0]
            if s == 0:
                want = 0
            assert q == want, (n, j, q, cands)


def test_scale_is_the_fp16_nearest_to_absmax_over_7():
    W = inputs.weight(32, 512, workload=73)
    perm = np.arange(512, dtype=np.int32)
    r = quantize_int4(W, perm, 0)
    amax = np.abs(W.astype(np.float64)).reshape(32, 16, 32).max(axis=2)
    for (n, g), s in np.ndenumerate(r["s"]):
        exact = Fraction(float(amax[n, g])) / 7
        assert abs(Fraction(float(s)) - exact) <= Fraction(_fp16_ulp(s)) / 2


def test_constructed_groups_are_recovered_exactly():
    """w = s0 * q0 with an fp16 s0 and integers |q0| <= 7 reaching 7 in every
    group: absmax / 7 = s0 exactly, so the codes and scales come back."""
    rng = np.random.default_rng(74)
    N, K = 8, 256
    s0 = np.float16(rng.uniform(1e-4, 1e-1, (N, K // 32)).astype(np.float16))
    q0 = rng.integers(-7, 8, (N, K)).astype(np.int8)
    q0[:, ::32] = 7 * np.where(rng.random((N, K // 32)) < 0.5, -1, 1)
    W = (np.repeat(s0.astype(np.float64), 32, axis=1) * q0).astype(np.float32)
    assert np.array_equal(W.astype(np.float64), np.repeat(s0.astype(np.float64), 32, axis=1) * q0)
    r = quantize_int4(W, np.arange(K, dtype=np.int32), 0)
    np.testing.assert_array_equal(r["q"], q0)
    np.testing.assert_array_equal(r["s"].view(np.uint16), s0.view(np.uint16))


def test_sign_symmetry_zero_groups_and_anchors():
    W = inputs.weight(16, 256, workload=75)
    W[:, 64:96] = 0.0          # a zero group in original order
    perm = np.arange(256, dtype=np.int32)[::-1].copy()
    n_out = 5
    r = quantize_int4(W, perm, n_out)
    rn = quantize_int4(-W, perm, n_out)
    np.testing.assert_array_equal(rn["q"], -r["q"])
    np.testing.assert_array_equal(rn["s"], r["s"])
    # original 64..95 sit at permuted positions 160..191: group 5
    assert np.all(r["s"][:, 5] == 0) and np.all(r["q"][:, 160:192] == 0)
    # anchors: fp16 of the original columns perm[0..n_out), codes zero there
    for o in range(n_out):
        c = int(perm[o])
        np.testing.assert_array_equal(r["W_O"][:, o], W[:, c].astype(np.float16))
    assert np.all(r["q"][:, :n_out] == 0)
    assert np.all(np.abs(r["q"]) <= 7)


def test_pack_nibble_layout_and_round_trip():
    q = np.array([[-7, 7, 0, -1, 3, -8 + 1, 2, 5]], np.int8)
    b = pack_int4(q)
    # nibbles q + 8: (1, 15) (8, 7) (11, 1) (10, 13), even position low
    np.testing.assert_array_equal(b, np.array([[0xF1, 0x78, 0x1B, 0xDA]], np.uint8))
    every = np.arange(256, dtype=np.uint8).reshape(4, 64)
    np.testing.assert_array_equal(pack_int4(unpack_int4(every)), every)
    qr = np.random.default_rng(76).integers(-7, 8, (5, 96)).astype(np.int8)
    np.testing.assert_array_equal(unpack_int4(pack_int4(qr)), qr)


def _brute_gemv(x_p, packed, s, W_O):
    """Double loop with exact rationals, decoding straight from the bytes."""
    B, K = x_p.shape
    N = packed.shape[0]
    n_out = W_O.shape[1]
    y = np.zeros((B, N))
    for b in range(B):
        for n in range(N):
            acc = Fraction(0)
            for j in range(K):
                byte = int(packed[n, j // 2])
                u = (byte >> (4 * (j % 2))) & 15
                w = Fraction(float(s[n, j // 32])) * (u - 8)
                if j < n_out:
                    w = Fraction(float(W_O[n, j]))
                acc += Fraction(float(x_p[b, j])) * w
            y[b, n] = float(acc)
    return y


def test_gemv_against_brute_force_and_unpermuted_weights():
    N, K, B, n_out = 3, 64, 2, 2
    W = inputs.weight(N, K, workload=77)
    Xp = inputs.profile(16, K, workload=77)
    perm = int4_permutation(W, Xp)
    r = quantize_int4(W, perm, n_out)
    x = inputs.act_f16(B, K, workload=77)
    x_p = permute_cols(x, perm)
    y = gemv_int4_ref(x_p, r["q"], r["s"], r["W_O"])
    np.testing.assert_allclose(y, _brute_gemv(x_p, pack_int4(r["q"]), r["s"], r["W_O"]), rtol=1e-13, atol=1e-15)
    # the same product in the original channel order: un-permute the weights
    Wo = np.zeros((N, K))
    wp = dequant_int4(r["q"], r["s"])
    wp[:, :n_out] = r["W_O"].astype(np.float64)
    Wo[:, perm] = wp
    np.testing.assert_allclose(y, x.astype(np.float64) @ Wo.T, rtol=1e-12, atol=1e-15)


def test_gemv_one_hot_reads_one_permuted_column():
    N, K, n_out = 5, 128, 3
    W = inputs.weight(N, K, workload=78)
    perm = np.random.default_rng(78).permutation(K).astype(np.int32)
    r = quantize_int4(W, perm, n_out)
    for j in (0, 2, 3, 31, 32, 127):
        x = np.zeros((1, K), np.float16)
        x[0, j] = 1
        y = gemv_int4_ref(x, r["q"], r["s"], r["W_O"])[0]
        want = r["W_O"][:, j].astype(np.float64) if j < n_out else \
            r["s"][:, j // 32].astype(np.float64) * r["q"][:, j]
        np.testing.assert_array_equal(y, want)


def test_prefill_weights_match_torch_bf16_cast():
    import torch
    W = inputs.weight(12, 256, workload=79)
    perm = np.arange(256, dtype=np.int32)
    r = quantize_int4(W, perm, 4)
    bits = prefill_weight_bf16_int4(r["q"], r["s"], r["W_O"])
    w32 = (np.repeat(r["s"].astype(np.float32), 32, axis=1) * r["q"].astype(np.float32))
    w32[:, :4] = r["W_O"].astype(np.float32)
    want = torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, want)


def test_int4_error_is_below_the_2bit_code_on_gaussian_weights():
    """Direction only: sixteen uniform levels per group beat four fitted
    levels on Gaussian weights (relative MSE, no anchors on either side)."""
    W = inputs.weight(64, 1024, workload=80)
    r4 = quantize_int4(W, np.arange(1024, dtype=np.int32), 0)
    e4 = np.mean((dequant_int4(r4["q"], r4["s"]) - W) ** 2) / np.mean(W.astype(np.float64) ** 2)
    r2 = oracle.quantize_2bit(W)
    e2 = np.mean((oracle.dequant_2bit(r2["q"], r2["S"], r2["Z"]) - W) ** 2) / np.mean(W.astype(np.float64) ** 2)
    print(f"relative MSE: int4 {e4:.4f}, 2-bit {e2:.4f}")
    assert e4 < e2 / 4
