"""Reference products against the quantized weights, in fp64.

The pages give no worked example of the products; they describe the kernel
as multiplying directly against the packed weights, decoding them in
registers ("Key v4.0 Innovations" of "On-The-Fly Weight Synthesizer
(OTF-LLM Engine v4.0)"). Mathematically the product is the plain one against
the dequantized matrix, which is what is written out here:

* decode GEMV (2-bit): y = x_R . W_hat^T + x[:, idx] . W_O^T, where x_R is x
  with the outlier channels zeroed (they are carried by the fp16 anchors
  W_O, section 4) and W_hat = S * C[q] + Z (section 3);
* decode GEMV (NF4): y = x . W_hat^T with W_hat = absmax * L[q];
* prefill GEMM: Y = X . W_bf16^T, where W_bf16 is the dequantized weight
  rounded once to fp32 (S*C+Z as one fused multiply-add, or absmax*L as one
  multiply) and then once to bf16, the precision the matrix cores consume;
  anchor columns carry their fp16 value rounded to bf16.

Inputs are taken exactly: fp16 / bf16 values widen to fp64 without error.
Matrix products use numpy's fp64 matmul as a library primitive.
"""

import numpy as np

from .codebook import CODEBOOK, CODEBOOK_F32
from .quant2bit import GROUP_2BIT, dequant_2bit
from .nf4 import BLOCK_NF4, nf4_levels, dequant_nf4
from .rounding import f32_to_bf16_rne_bits, bf16_bits_to_f64


def gemv_2bit_ref(x16, q, S, Z, idx=None, W_O=None):
    x64 = np.asarray(x16, dtype=np.float16).astype(np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    W_hat = dequant_2bit(q, S, Z)
    xR = x64.copy()
    y = None
    if idx is not None and len(idx):
        idx = np.asarray(idx, dtype=np.int64)
        xR[:, idx] = 0.0
        y = x64[:, idx] @ np.asarray(W_O, np.float16).astype(np.float64).T
    base = xR @ W_hat.T
    return base if y is None else base + y


def gemv_nf4_ref(x16, q, absmax):
    x64 = np.asarray(x16, dtype=np.float16).astype(np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    return x64 @ dequant_nf4(q, absmax).T


def _fl32_of_exact_sum(p, z):
    """Round the exact sum p + z (fp64 operands) once to fp32.

    TwoSum gives s + e == p + z exactly. Rounding s alone is right unless s
    lies exactly on the midpoint between two fp32 neighbours while e != 0;
    then the exact value is on the side of sign(e), and that neighbour is
    the result.
    """
    p = np.asarray(p, np.float64)
    z = np.asarray(z, np.float64)
    s = p + z
    bp = s - p
    e = (p - (s - bp)) + (z - bp)
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(-np.inf))
    mid_up = s == 0.5 * (r64 + up.astype(np.float64))
    mid_dn = s == 0.5 * (r64 + dn.astype(np.float64))
    hi = np.where(mid_up, up, r)
    lo = np.where(mid_dn, dn, r)
    on_mid = mid_up | mid_dn
    out = np.where(on_mid & (e > 0), hi, np.where(on_mid & (e < 0), lo, r))
    return out.astype(np.float32)


def prefill_weight_bf16_2bit(q, S, Z, idx=None, W_O=None):
    """bf16 bit patterns of the dequantized 2-bit weights as the prefill GEMM
    consumes them: bf16(fl32(S*C[q] + Z)); anchor columns hold bf16(W_O)."""
    q = np.asarray(q)
    S64 = np.repeat(np.asarray(S, np.float64), GROUP_2BIT, axis=1)
    Z64 = np.repeat(np.asarray(Z, np.float64), GROUP_2BIT, axis=1)
    p = S64 * CODEBOOK[q]                  # exact: 11-bit x 24-bit
    w32 = _fl32_of_exact_sum(p, Z64)
    bits = f32_to_bf16_rne_bits(w32)
    if idx is not None and len(idx):
        a32 = np.asarray(W_O, np.float16).astype(np.float32)
        bits[:, np.asarray(idx, np.int64)] = f32_to_bf16_rne_bits(a32)
    return bits


def prefill_weight_bf16_nf4(q, absmax):
    """bf16(fl32(absmax * L[q])); the fp32 product is exact in fp64."""
    L = nf4_levels().astype(np.float64)
    a = np.repeat(np.asarray(absmax, np.float64), BLOCK_NF4, axis=1)
    w32 = (a * L[np.asarray(q)]).astype(np.float32)
    return f32_to_bf16_rne_bits(w32)


def gemm_prefill_ref(X_bf16_bits, W_bf16_bits):
    """Y = X . W^T in fp64 from bf16 bit patterns of X (M, K) and W (N, K)."""
    X = bf16_bits_to_f64(X_bf16_bits)
    W = bf16_bits_to_f64(W_bf16_bits)
    return X @ W.T
