"""The adaptive non-uniform 2-bit code: quantize, pack, unpack, dequantize.

Source: "On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)":
* "Key v4.0 Innovations": Lloyd-Max Gaussian centroids, closed-form linear
  regression per group of G=32, four 2-bit weights per uint8.
* Section 3 ("Closed-Form Group Linear Regression"): least squares fit of
  W_g ~ S_g * C[q_i] + Z_g with the printed closed form for S_g (centred
  cross-product over centred sum of squares plus epsilon) and
  Z_g = mean(W_g) - S_g * mean(C_q).
* Section 4 ("Profile-Guided Activation Outliers"): the top-scoring input
  channels are kept exactly in FP16 outside the 2-bit code.

Readings taken where the page is silent (each one is also listed with the
design notes):
* groups run along K inside one row; K must be a multiple of 32;
* how codes are assigned before the fit is not stated. The codebook is the
  N(0,1)-optimal one, so each group is standardised by its own mean and
  population standard deviation and each weight takes the nearest centroid;
  a single pass, then the fit. With symmetric levels the nearest-centroid
  rule is: sign of (w - mean) picks the half, and |w - mean| > t*sigma with
  t = (C[2] + C[3]) / 2 picks the outer level. Written without square root
  or division as (w - mean)^2 > t^2 * var. A deviation of exactly 0 goes to
  the upper half; a tie on the outer threshold goes to the inner level;
  a constant group therefore gets code 2 everywhere, S = 0 and Z = mean;
* epsilon in the denominator is 1e-8;
* S and Z are stored as fp16, each rounded once from the fp64 result; Z is
  computed from the unrounded S, as the formula is printed;
* every in-group sum is sequential, left to right, in fp64, with no fused
  multiply-add;
* outlier columns are zeroed before quantizing (the full-K layout is kept,
  their codes are stored but never used) and their fp32 weights are kept as
  fp16 anchors.

Optional refinement (a variant of the same format, off by default): the
section-3 fit takes the codes as given, and section 2 picks each code as the
nearest centroid. Alternating the two on the fitted levels lowers the
group's squared error further, as in Lloyd's method. One round:
* levels l_j = S * C[j] + Z from the unrounded fit (fp64, product then sum);
* each weight moves to the level nearest to it, |w - l_j| in fp64; a weight
  whose current level is among the nearest keeps its code, otherwise the
  lowest nearest j is taken;
* the fit is redone with the new codes exactly as above (same mean m and
  deviations d, same sums, same epsilon).
A round that changes no code leaves S and Z unchanged, so every later round
does too. S and Z of the last fit are rounded to fp16.
"""

import numpy as np

from .codebook import CODEBOOK, CODEBOOK_F32
from .rounding import fp16_rne

GROUP_2BIT = 32
OLS_EPS = 1e-8


def _seq_sum(a):
    """Sequential left-to-right fp64 sum over the last axis (length 32)."""
    acc = np.zeros(a.shape[:-1], dtype=np.float64)
    for i in range(a.shape[-1]):
        acc = acc + a[..., i]
    return acc


def assign_codes_2bit(d, var):
    """Nearest standardised centroid for deviations ``d`` (..., 32) of groups
    with population variance ``var`` (...). Returns codes 0..3 (uint8)."""
    t = 0.5 * (CODEBOOK[2] + CODEBOOK[3])
    thr = (t * t) * var[..., None]
    outer = (d * d) > thr
    upper = d >= 0.0
    q = np.where(upper, np.where(outer, 3, 2), np.where(outer, 0, 1))
    return q.astype(np.uint8)


def _ols(d, m, q):
    """Section-3 fit for codes ``q`` given deviations ``d`` = w - m."""
    c = CODEBOOK[q]
    cbar = _seq_sum(c) / GROUP_2BIT
    cc = c - cbar[..., None]
    num = _seq_sum(d * cc)
    den = _seq_sum(cc * cc) + OLS_EPS
    S = num / den
    Z = m - S * cbar
    return S, Z


def reassign_nearest_2bit(g, q, S, Z):
    """Codes of the levels S*C[j] + Z nearest to each weight of ``g`` (..., 32);
    ties keep the current code ``q`` when it is among the nearest, else take
    the lowest j."""
    lev = S[..., None] * CODEBOOK + Z[..., None]              # (..., 4)
    dist = np.abs(g[..., :, None] - lev[..., None, :])         # (..., 32, 4)
    best = dist.min(axis=-1)
    cur = np.take_along_axis(dist, q[..., None].astype(np.int64), axis=-1)[..., 0]
    first = np.argmax(dist == best[..., None], axis=-1)
    return np.where(cur == best, q, first).astype(np.uint8)


def fit_2bit_groups(g, refine_rounds=0):
    """Codes and unrounded fp64 (S, Z) for fp64 groups ``g`` (..., 32), after
    ``refine_rounds`` rounds of reassignment and refit."""
    m = _seq_sum(g) / GROUP_2BIT
    d = g - m[..., None]
    var = _seq_sum(d * d) / GROUP_2BIT
    q = assign_codes_2bit(d, var)
    S, Z = _ols(d, m, q)
    for _ in range(int(refine_rounds)):
        q = reassign_nearest_2bit(g, q, S, Z)
        S, Z = _ols(d, m, q)
    return q, S, Z


def quantize_2bit(W, outlier_idx=None, refine_rounds=0):
    """Quantize fp32 ``W`` (N, K) to the 2-bit group code (``refine_rounds``
    rounds of reassignment and refit after the single pass).

    Returns a dict with
      q   : uint8 (N, K) codes 0..3 (unpacked),
      S, Z: float16 (N, K/32) per-group scale and offset,
      idx : int32 (n_out,) ascending outlier channels,
      W_O : float16 (N, n_out) exact-fp16 anchors (columns idx of W).
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if K % GROUP_2BIT:
        raise ValueError("K must be a multiple of 32")
    idx = np.zeros(0, np.int32) if outlier_idx is None else np.asarray(outlier_idx, np.int32)
    W64 = W.astype(np.float64)
    W_O = fp16_rne(W64[:, idx])
    if idx.size:
        W64[:, idx] = 0.0

    q, S, Z = fit_2bit_groups(W64.reshape(N, K // GROUP_2BIT, GROUP_2BIT), refine_rounds)
    return {
        "q": q.reshape(N, K),
        "S": fp16_rne(S),
        "Z": fp16_rne(Z),
        "idx": idx,
        "W_O": W_O,
    }


def pack_2bit(q):
    """Four codes per byte along K: byte j of a row holds the codes of
    elements 4j..4j+3, element 4j+t in bits 2t and 2t+1."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    r = q.reshape(N, K // 4, 4).astype(np.uint32)
    b = r[..., 0] | (r[..., 1] << 2) | (r[..., 2] << 4) | (r[..., 3] << 6)
    return b.astype(np.uint8)


def unpack_2bit(packed):
    """Inverse of ``pack_2bit``: (N, K/4) bytes -> (N, K) codes."""
    p = np.asarray(packed, dtype=np.uint8)
    N, KB = p.shape
    out = np.empty((N, KB, 4), dtype=np.uint8)
    for t in range(4):
        out[..., t] = (p >> (2 * t)) & 3
    return out.reshape(N, KB * 4)


def dequant_2bit(q, S, Z):
    """w_hat[n, k] = S[n, g] * C[q[n, k]] + Z[n, g] (g = k // 32), in fp64
    from the stored fp16 S, Z and the fp32 codebook constants."""
    q = np.asarray(q)
    N, K = q.shape
    S64 = np.repeat(np.asarray(S, np.float64), GROUP_2BIT, axis=1)
    Z64 = np.repeat(np.asarray(Z, np.float64), GROUP_2BIT, axis=1)
    return S64 * CODEBOOK[q] + Z64


def sz_interleaved(S, Z):
    """(S, Z) as the stored pairs: float16 (N, K/32, 2) with [..., 0] = S."""
    return np.stack([np.asarray(S, np.float16), np.asarray(Z, np.float16)], axis=-1)


__all__ = ["GROUP_2BIT", "OLS_EPS", "CODEBOOK_F32", "assign_codes_2bit", "fit_2bit_groups",
           "reassign_nearest_2bit",
           "quantize_2bit", "pack_2bit", "unpack_2bit", "dequant_2bit",
           "sz_interleaved"]
