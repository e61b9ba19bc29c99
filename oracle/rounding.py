"""Rounding to the storage types used by the formats.

* fp64 -> fp16: one direct round-to-nearest-even, subnormals kept. numpy's
  ``astype(np.float16)`` from float64 rounds directly (it does not pass
  through fp32); tests pin that on hand-derived bit patterns, including a
  value that double rounding through fp32 would get wrong.
* fp32 -> bf16: round-to-nearest-even on the bit pattern, written out here.
"""

import numpy as np


def fp16_rne(x):
    """Direct fp64 -> fp16 round-to-nearest-even of ``x`` (array-like)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16)


def f32_to_bf16_rne_bits(x32):
    """fp32 -> bf16 round-to-nearest-even; returns the uint16 bit patterns.

    bf16 keeps the top 16 bits of the fp32 pattern. The dropped low half is
    compared with 0x8000: above rounds up, below rounds down, equal rounds to
    the even kept pattern. A carry out of the mantissa bumps the exponent,
    which is the right result (up to infinity). NaNs stay quiet NaNs.
    """
    b = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = b >> np.uint64(16)
    low = b & np.uint64(0xFFFF)
    up = (low > 0x8000) | ((low == 0x8000) & ((keep & np.uint64(1)) == 1))
    out = keep + up.astype(np.uint64)
    isnan = np.isnan(np.asarray(x32, dtype=np.float32))
    out = np.where(isnan, keep | np.uint64(0x0040), out)
    return out.astype(np.uint16)


def bf16_bits_to_f64(bits):
    """Exact widening of bf16 bit patterns to fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)
