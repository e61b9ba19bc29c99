"""The 2-bit codebook and the Lloyd-Max quantizer it comes from.

Source: "On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)", section 2
("Why Uniform Linear 2-Bit Quantization Fails" / "The Lloyd-Max Non-Uniform
Solution"). The page states the mean squared quantization error objective
over the four cells of a normal density and prints the resulting four-level
codebook to two decimals. The printed decimals, rounded to fp32, are the format
constant; the Lloyd iteration below exists to pin them.
"""

import numpy as np
from scipy.stats import norm

# The four centroids as printed on the page (section 2), ascending, as fp32.
CODEBOOK_F32 = np.array([-1.52, -0.45, 0.45, 1.52], dtype=np.float32)
# The same constants promoted exactly to fp64.
CODEBOOK = CODEBOOK_F32.astype(np.float64)


def _cell_moments(a, b):
    """Zeroth, first and second moments of N(0,1) restricted to [a, b].

    Closed forms: P = Phi(b) - Phi(a); int w phi = phi(a) - phi(b);
    int w^2 phi = P + a phi(a) - b phi(b) (integration by parts), with the
    a*phi(a) term taken as 0 at an infinite end.
    """
    P = norm.cdf(b) - norm.cdf(a)
    m1 = norm.pdf(a) - norm.pdf(b)
    ta = 0.0 if np.isinf(a) else a * norm.pdf(a)
    tb = 0.0 if np.isinf(b) else b * norm.pdf(b)
    m2 = P + ta - tb
    return P, m1, m2


def _thresholds(levels):
    """Nearest-neighbour cell boundaries: midpoints, with -inf and +inf ends."""
    c = np.asarray(levels, dtype=np.float64)
    return np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))


def gaussian_msqe(levels):
    """The section-2 objective: sum over cells of int (w - c_q)^2 p(w) dw for
    p = N(0,1), with each cell the nearest-neighbour region of its level."""
    c = np.asarray(levels, dtype=np.float64)
    t = _thresholds(c)
    total = 0.0
    for q in range(len(c)):
        P, m1, m2 = _cell_moments(t[q], t[q + 1])
        total += m2 - 2.0 * c[q] * m1 + c[q] * c[q] * P
    return total


def lloyd_max_gaussian(init, iters=1000, tol=1e-15):
    """Lloyd's alternation for N(0,1): thresholds at the midpoints of the
    current levels, then each level moved to the conditional mean of its cell.

    Returns (levels, thresholds, msqe, iterations_used).
    """
    c = np.sort(np.asarray(init, dtype=np.float64))
    used = 0
    for used in range(1, iters + 1):
        t = _thresholds(c)
        new = np.empty_like(c)
        for q in range(len(c)):
            P, m1, _ = _cell_moments(t[q], t[q + 1])
            new[q] = m1 / P
        step = np.max(np.abs(new - c))
        c = new
        if step < tol:
            break
    return c, _thresholds(c)[1:-1], gaussian_msqe(c), used
