"""Profile-guided outlier anchor selection.

Source: "On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)", section 4
("Profile-Guided Activation Outliers"): a calibration pass records the mean
activation magnitude of each input channel; the channel impact score is a
column norm of W times that magnitude; the top 3.5% channels are kept in
FP16. The page writes the score two ways: the section-4 equation uses the
column 2-norm, while the title and the feature list use the shorthand
|W| x |X_profile|. Both are provided:

* ``SCORE_MEANABS``: mean over rows of |W[:, c]| times mean |X_profile[:, c]|
  (the |W| x |X| shorthand read as mean magnitudes);
* ``SCORE_L2``: ||W[:, c]||_2 times mean |X_profile[:, c]| (the equation).

Readings: the number kept is floor(frac * K) computed in fp64; sums over rows
are sequential in fp64; the sort is by descending score, ties to the lower
channel; the result is returned ascending.
"""

import math

import numpy as np

SCORE_MEANABS = 1
SCORE_L2 = 2


def outlier_count(K, frac):
    return int(math.floor(float(frac) * float(K)))


def _seq_row_sum(a):
    """Sequential fp64 sum over axis 0 (rows), one column at a time in
    parallel."""
    acc = np.zeros(a.shape[1], dtype=np.float64)
    for r in range(a.shape[0]):
        acc = acc + a[r]
    return acc


def profile_abs_sum(Xp):
    """Sum over calibration rows of |X[:, c]| (fp64, rows added in order)."""
    X64 = np.asarray(Xp, dtype=np.float32).astype(np.float64)
    return _seq_row_sum(np.abs(X64))


def profile_absmean(Xp):
    """Mean over calibration rows of |X[:, c]| (fp64, sequential)."""
    return profile_abs_sum(Xp) / np.asarray(Xp).shape[0]


def channel_scores(W, Xp, kind=SCORE_MEANABS):
    W64 = np.asarray(W, dtype=np.float32).astype(np.float64)
    pm = profile_absmean(Xp)
    if kind == SCORE_MEANABS:
        col = _seq_row_sum(np.abs(W64)) / W64.shape[0]
    elif kind == SCORE_L2:
        col = np.sqrt(_seq_row_sum(W64 * W64))
    else:
        raise ValueError("unknown score kind")
    return col * pm


def select_outliers(W, Xp, frac, kind=SCORE_MEANABS):
    """Top floor(frac*K) channels by score, returned ascending (int32)."""
    s = channel_scores(W, Xp, kind)
    K = s.shape[0]
    n = outlier_count(K, frac)
    order = sorted(range(K), key=lambda c: (-s[c], c))
    return np.array(sorted(order[:n]), dtype=np.int32)
