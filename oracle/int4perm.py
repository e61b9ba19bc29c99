"""The v3.2 INT4 permutation format: quantize, pack, unpack, dequantize, and
the products against it.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check
and the benchmark's CPU baseline use it.

Source: "On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)", "Comparative
Analysis: INT4 (v3.2) vs INT2 Non-Uniform (v4.0)" and its "Method Comparison
Table": two 4-bit weights per byte, a uniform linear grid, a symmetric grid
with zero-point 0, a global static permutation of the channels
(``global_perm_idx``), and the top 1% channels by a weight-activation score
kept in FP16.

The page gives no group size, scale type, rounding rule, nor how the
permutation is chosen or used. Readings taken (each one is also listed with
the design notes):

* permutation: the input channels ordered by descending outlier score (the
  weight-activation score of section 4, the same function as the 2-bit
  anchors), ties to the lower channel; ``perm[j]`` is the channel at
  permuted position j. "Global" is read as: the channel space is reordered
  once, so activations arrive in permuted order, ``x_p[:, j] = x[:,
  perm[j]]``, and the products take them that way;
* anchors: the first n_out = floor(0.01 K) permuted channels (the top 1%)
  are kept exactly as fp16 weights W_O; their INT4 columns are zeroed before
  quantization, so they hold the zero level;
* grid: levels s * q with q in -7..7 (symmetric about 0; the 16th code is
  unused), one fp16 scale per group of 32 consecutive permuted channels of a
  row: s = fp16(absmax / 7) (absmax after zeroing the anchors; the quotient
  in fp64, one round-to-nearest-even to fp16), and
  q = clamp(round-half-even(w / s), -7, 7) in fp64 with the stored s, so
  that s * q is the nearest grid level to w; s = 0 gives q = 0;
* storage: nibble u = q + 8; two per byte, the even permuted position in
  the low nibble.
"""

import numpy as np

from .outliers import SCORE_MEANABS, channel_scores
from .rounding import fp16_rne, f32_to_bf16_rne_bits

GROUP_INT4 = 32
QMAX_INT4 = 7
ANCHOR_FRAC_INT4 = 0.01


def int4_permutation(W, Xp, kind=SCORE_MEANABS):
    """Channels by descending score (ties: lower channel first), int32 [K]."""
    s = channel_scores(W, Xp, kind)
    K = s.shape[0]
    order = sorted(range(K), key=lambda c: (-s[c], c))
    return np.array(order, dtype=np.int32)


def permute_cols(A, perm):
    """Columns of A (M, K) in permuted order: out[:, j] = A[:, perm[j]]."""
    return np.asarray(A)[:, np.asarray(perm, np.int64)]


def quantize_int4(W, perm, n_out):
    """Quantize fp32 W (N, K) in its original channel order.

    Returns a dict with
      q    int8 [N][K]   codes -7..7 in permuted order (0 at the anchors)
      s    fp16 [N][K/32] group scales
      W_O  fp16 [N][n_out] anchor weights (permuted positions 0..n_out-1)
      perm int32 [K]
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if K % GROUP_INT4:
        raise ValueError("K must be a multiple of 32")
    perm = np.asarray(perm, np.int32)
    if sorted(perm.tolist()) != list(range(K)):
        raise ValueError("perm must be a permutation of 0..K-1")
    if not 0 <= n_out < K:
        raise ValueError("n_out out of range")
    Wp = permute_cols(W, perm).astype(np.float64)
    W_O = fp16_rne(Wp[:, :n_out])
    Wp[:, :n_out] = 0.0
    G = K // GROUP_INT4
    g = Wp.reshape(N, G, GROUP_INT4)
    absmax = np.max(np.abs(g), axis=2)
    s16 = fp16_rne(absmax / QMAX_INT4)
    s64 = s16.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s64 > 0, g / np.where(s64 > 0, s64, 1.0), 0.0)
    q = np.clip(np.rint(r), -QMAX_INT4, QMAX_INT4).astype(np.int8)
    return {"q": q.reshape(N, K), "s": s16, "W_O": W_O, "perm": perm}


def pack_int4(q):
    """Codes -7..7 (N, K) -> uint8 (N, K/2): nibble q + 8, even position low."""
    u = (np.asarray(q, np.int16) + 8).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(codes):
    """uint8 (N, K/2) -> codes int8 (N, K)."""
    c = np.asarray(codes, np.uint8)
    lo = (c & 0x0F).astype(np.int16) - 8
    hi = (c >> 4).astype(np.int16) - 8
    out = np.empty((c.shape[0], 2 * c.shape[1]), np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def dequant_int4(q, s):
    """w_hat = s * q in fp64, permuted order (N, K)."""
    s64 = np.repeat(np.asarray(s, np.float16).astype(np.float64), GROUP_INT4, axis=1)
    return s64 * np.asarray(q, np.float64)


def gemv_int4_ref(x16_perm, q, s, W_O):
    """y = x_p . w_hat^T + x_p[:, :n_out] . W_O^T in fp64, with x_p the fp16
    activations in permuted channel order (the anchor columns of w_hat are
    zero)."""
    x = np.asarray(x16_perm, np.float16).astype(np.float64)
    if x.ndim == 1:
        x = x[None, :]
    W_O = np.asarray(W_O, np.float16).astype(np.float64)
    y = x @ dequant_int4(q, s).T
    n_out = W_O.shape[1]
    if n_out:
        y = y + x[:, :n_out] @ W_O.T
    return y


def prefill_weight_bf16_int4(q, s, W_O):
    """bf16 bit patterns (permuted order) of the weights the prefill GEMM
    consumes: bf16(s * q) (the product is exact in fp32), anchor columns
    bf16(W_O)."""
    w32 = dequant_int4(q, s).astype(np.float32)  # exact: 11-bit x 4-bit
    bits = f32_to_bf16_rne_bits(w32)
    W_O = np.asarray(W_O, np.float16)
    if W_O.shape[1]:
        bits[:, :W_O.shape[1]] = f32_to_bf16_rne_bits(W_O.astype(np.float32))
    return bits
