"""NF4 (NormalFloat4) block-wise weight quantization.

Source: "AirQuant" README, "Fundamentacao Teorica e Arquitetura" item 2
(bitsandbytes NormalFloat4 with block-wise precision, about a quarter of the
FP16 footprint) and "Fontes" (QLoRA, Dettmers et al. 2023, as the formal
basis of NF4). The pages give neither the 16 levels nor the block size, so:

* levels (reading of the QLoRA construction): quantiles of N(0,1), 8 on the
  positive side at probabilities evenly spaced from delta down to 1/2
  (1/2 itself excluded), 7 on the negative side the same way, plus an exact
  zero; all divided by the largest so they span [-1, 1]. delta puts the
  outermost level half a step in from the tail, averaged over the 16-level
  and 15-level spacings: delta = 1 - (1/32 + 1/30) / 2. Computed in fp64 and
  rounded once to fp32;
* blocks of 64 consecutive weights along K inside one row, with an fp32
  absmax per block;
* a weight w of a block with absmax a > 0 takes the level nearest to w / a,
  a tie going to the lower level; written exactly as the count of midpoints
  t_j = (L_j + L_{j+1}) / 2 with w > t_j * a (both products exact in fp64);
* an all-zero block stores absmax 0 and code 7 (the zero level);
* two codes per byte, the even element in the low nibble.
"""

import numpy as np
from scipy.special import ndtri

BLOCK_NF4 = 64
NF4_DELTA = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)


def nf4_levels():
    """The 16 NF4 levels, ascending, as fp32."""
    pos = ndtri(np.linspace(NF4_DELTA, 0.5, 9)[:-1])      # 8 positive
    neg = -ndtri(np.linspace(NF4_DELTA, 0.5, 8)[:-1])     # 7 negative
    v = np.sort(np.concatenate([neg, [0.0], pos]))
    v = v / np.max(v)
    return v.astype(np.float32)


def quantize_nf4(W):
    """Quantize fp32 ``W`` (N, K) to NF4. Returns (q uint8 (N, K) in 0..15,
    absmax float32 (N, K/64))."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if K % BLOCK_NF4:
        raise ValueError("K must be a multiple of 64")
    L = nf4_levels().astype(np.float64)
    mids = 0.5 * (L[:-1] + L[1:])
    blocks = W.reshape(N, K // BLOCK_NF4, BLOCK_NF4)
    a = np.max(np.abs(blocks), axis=-1)                    # exact in fp32
    w64 = blocks.astype(np.float64)
    a64 = a.astype(np.float64)[..., None]
    q = np.zeros(blocks.shape, dtype=np.uint8)
    for j in range(15):
        q += (w64 > mids[j] * a64).astype(np.uint8)
    q = np.where(a64 == 0.0, np.uint8(7), q)
    return q.reshape(N, K), a.astype(np.float32)


def pack_nf4(q):
    """Two codes per byte: byte j holds element 2j (low nibble) and 2j+1."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    r = q.reshape(N, K // 2, 2)
    return (r[..., 0] | (r[..., 1] << 4)).astype(np.uint8)


def unpack_nf4(packed):
    p = np.asarray(packed, dtype=np.uint8)
    N, KB = p.shape
    out = np.empty((N, KB, 2), dtype=np.uint8)
    out[..., 0] = p & 15
    out[..., 1] = p >> 4
    return out.reshape(N, KB * 2)


def dequant_nf4(q, absmax):
    """w_hat = absmax[block] * L[q] in fp64 (the product of two fp32 values,
    exact in fp64)."""
    L = nf4_levels().astype(np.float64)
    a = np.repeat(np.asarray(absmax, np.float64), BLOCK_NF4, axis=1)
    return a * L[np.asarray(q)]
