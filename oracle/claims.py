"""Checks of the pages' quantitative claims that are not part of the format.

"On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)", section 2, says that
a uniform 2-bit grid spanning W_min..W_max wastes levels on the tails, and
that the Lloyd-Max codebook lowers the MSE "4.2x" against such a grid. The
page does not say on which data, group size or fit. Parity unpinned: this
module only measures the ratio on a stated setting; nothing is gated on it.
"""

import numpy as np

from .quant2bit import quantize_2bit, dequant_2bit, GROUP_2BIT


def uniform_minmax_2bit(W):
    """Per group of 32 along K: four evenly spaced levels from the group
    minimum to its maximum, each weight to the nearest level."""
    W64 = np.asarray(W, np.float32).astype(np.float64)
    N, K = W64.shape
    g = W64.reshape(N, K // GROUP_2BIT, GROUP_2BIT)
    lo = g.min(axis=-1, keepdims=True)
    hi = g.max(axis=-1, keepdims=True)
    step = (hi - lo) / 3.0
    safe = np.where(step > 0, step, 1.0)
    q = np.clip(np.rint((g - lo) / safe), 0, 3)
    return (lo + q * step).reshape(N, K)


def uniform_vs_lloyd_mse_ratio(W):
    """MSE(uniform min-max grid) / MSE(Lloyd-Max codebook + OLS fit) on W."""
    W64 = np.asarray(W, np.float32).astype(np.float64)
    r = quantize_2bit(W)
    ours = dequant_2bit(r["q"], r["S"], r["Z"])
    uni = uniform_minmax_2bit(W)
    return float(np.mean((uni - W64) ** 2) / np.mean((ours - W64) ** 2))
