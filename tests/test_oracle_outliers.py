"""Pins of the outlier selection (oracle/outliers.py): scores against numpy's
own column reductions, the selection against an independent lexicographic
sort, and the selection's defining property (every kept score >= every
dropped score)."""

import json
import os

import numpy as np
import pytest

from oracle import (outlier_count, profile_absmean, channel_scores,
                    select_outliers, SCORE_MEANABS, SCORE_L2)
from bit_weight_quantized_qw_amd import inputs


def test_count_rounding(golden_dir):
    with open(os.path.join(golden_dir, "pages_figures.json")) as f:
        frac = json.load(f)["outlier_frac"]["value"]
    assert outlier_count(5120, frac) == 179
    assert outlier_count(27648, frac) == 967
    assert outlier_count(2048, frac) == 71
    assert outlier_count(32, 0.0) == 0


@pytest.mark.parametrize("kind", [SCORE_MEANABS, SCORE_L2])
def test_scores_against_numpy(kind):
    W = inputs.weight(300, 512, workload=31)
    X = inputs.profile(64, 512, workload=31)
    s = channel_scores(W, X, kind)
    W64 = W.astype(np.float64)
    pm = np.mean(np.abs(X.astype(np.float64)), axis=0)
    col = np.mean(np.abs(W64), axis=0) if kind == SCORE_MEANABS else np.linalg.norm(W64, axis=0)
    np.testing.assert_allclose(s, col * pm, rtol=1e-13)
    np.testing.assert_allclose(profile_absmean(X), pm, rtol=1e-13)


@pytest.mark.parametrize("kind", [SCORE_MEANABS, SCORE_L2])
def test_selection_property_and_independent_sort(kind):
    W = inputs.weight(200, 1024, workload=32)
    X = inputs.profile(32, 1024, workload=32)
    idx = select_outliers(W, X, 0.035, kind)
    s = channel_scores(W, X, kind)
    n = outlier_count(1024, 0.035)
    assert idx.dtype == np.int32 and len(idx) == n
    assert np.all(np.diff(idx) > 0)
    mask = np.zeros(1024, bool)
    mask[idx] = True
    assert s[mask].min() >= s[~mask].max()
    ref = np.sort(np.lexsort((np.arange(1024), -s))[:n])
    np.testing.assert_array_equal(idx, ref)


def test_ties_go_to_lower_channel():
    W = np.ones((4, 64), np.float32)
    X = np.ones((2, 64), np.float32)
    idx = select_outliers(W, X, 0.1, SCORE_MEANABS)
    np.testing.assert_array_equal(idx, np.arange(6))


def test_spiked_channels_are_selected():
    # 14B-shaped workload: 1% of 5120 profile channels scaled x20
    K = 5120
    W = inputs.weight(1024, K, workload=3)
    X = inputs.profile(256, K, workload=3)
    ch = inputs.rng(3, 0, 0, inputs.ROLE_SPIKE).choice(K, 51, replace=False)
    for kind in (SCORE_MEANABS, SCORE_L2):
        idx = select_outliers(W, X, 0.035, kind)
        assert len(idx) == 179
        assert set(ch.tolist()) <= set(idx.tolist())
