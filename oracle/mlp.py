"""The gated activation between the gate/up and down projections of a
decoder block, in fp64. TEST INFRASTRUCTURE (see the package docstring).

The OTF-LLM page quantizes every projection of decoder blocks whose sizes it
quotes (3B to 32B models; the 32B class has hidden size 5120 and
intermediate size 27648), and its section 1 argues that decoding streams
every weight once per token, but it never names the activation between the
gate/up projections and the down projection. Reading taken: the gated SiLU
of that decoder family,

    x_down = silu(gate) * up,   silu(t) = t / (1 + exp(-t)),

with gate and up one linear map of their shared input: rows 0..I-1 (gate)
and I..2I-1 (up) of one merged 2I x K matrix, quantized as one matrix (one
anchor set chosen over both halves, section 4).
"""

import numpy as np

from .products import gemv_2bit_ref


def silu(t):
    """t * sigmoid(t) in fp64 (exp(-t) overflowing to inf for t below about
    -709 gives -0.0, the limit)."""
    t = np.asarray(t, np.float64)
    with np.errstate(over="ignore"):
        return t / (1.0 + np.exp(-t))


def swiglu_ref(y_merged):
    """silu(gate) * up from the outputs of a merged gate/up product, (..., 2I)
    -> (..., I), fp64."""
    y = np.asarray(y_merged, np.float64)
    if y.shape[-1] % 2:
        raise ValueError("a merged gate/up output has 2I values")
    i = y.shape[-1] // 2
    return silu(y[..., :i]) * y[..., i:]


def gemv_2bit_swiglu_ref(x16, q, S, Z, idx, W_O):
    """The merged gate/up GEMV against the 2-bit quantization of the merged
    matrix (gemv_2bit_ref), followed by the gated activation: (B, I) fp64."""
    return swiglu_ref(gemv_2bit_ref(x16, q, S, Z, idx, W_O))
