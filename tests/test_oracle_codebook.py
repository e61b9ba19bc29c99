"""Pins of the 2-bit codebook (oracle/codebook.py) against the Lloyd-Max
quantizer for N(0,1) -- the textbook result the page's section 2 invokes --
and against numerical quadrature, which shares nothing with the closed forms.
"""

import json
import os

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm

from oracle import CODEBOOK, CODEBOOK_F32, lloyd_max_gaussian, gaussian_msqe


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "pages_figures.json")) as f:
        return json.load(f)


def test_codebook_constant_is_the_printed_one(golden_dir):
    g = _golden(golden_dir)
    np.testing.assert_array_equal(CODEBOOK_F32, np.array(g["codebook"]["value"], np.float32))
    assert CODEBOOK.dtype == np.float64
    np.testing.assert_array_equal(CODEBOOK, CODEBOOK_F32.astype(np.float64))


@pytest.mark.parametrize("init", [
    [-3.0, -1.0, 1.0, 3.0],
    [-0.1, -0.05, 0.05, 0.1],
    [-2.0, -1.9, 0.3, 2.5],          # asymmetric start
])
def test_lloyd_converges_to_printed_codebook(init):
    c, t, mse, used = lloyd_max_gaussian(init, iters=5000)
    assert used < 5000
    # within the two printed decimals of the page
    assert np.max(np.abs(c - CODEBOOK)) < 0.01
    # symmetric solution with the middle threshold at 0
    assert abs(c[0] + c[3]) < 1e-9 and abs(c[1] + c[2]) < 1e-9
    assert abs(t[1]) < 1e-9


def test_lloyd_fixed_point_matches_max_table():
    # Max (1960), optimum 4-level quantizer for a unit normal:
    # outputs +-0.4528, +-1.510, threshold +-0.9816, distortion 0.1175.
    c, t, mse, _ = lloyd_max_gaussian([-1, -0.3, 0.3, 1], iters=5000)
    np.testing.assert_allclose(c, [-1.510, -0.4528, 0.4528, 1.510], atol=6e-4)
    np.testing.assert_allclose(t, [-0.9816, 0.0, 0.9816], atol=6e-4)
    assert abs(mse - 0.1175) < 1e-4


def test_fixed_point_conditions_by_quadrature():
    c, t, _, _ = lloyd_max_gaussian([-1, -0.3, 0.3, 1], iters=5000)
    edges = np.concatenate(([-np.inf], t, [np.inf]))
    for q in range(4):
        num = integrate.quad(lambda w: w * norm.pdf(w), edges[q], edges[q + 1])[0]
        den = integrate.quad(norm.pdf, edges[q], edges[q + 1])[0]
        assert abs(num / den - c[q]) < 1e-9     # centroid condition
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), atol=1e-15)  # midpoint condition


@pytest.mark.parametrize("levels", [
    list(CODEBOOK),
    [-1.5, -0.5, 0.5, 1.5],
    [-2.0, -0.1, 0.7, 1.1],
])
def test_msqe_closed_form_against_quadrature(levels):
    levels = np.asarray(levels, np.float64)
    edges = np.concatenate(([-np.inf], 0.5 * (levels[:-1] + levels[1:]), [np.inf]))
    ref = sum(integrate.quad(lambda w, c=levels[q]: (w - c) ** 2 * norm.pdf(w),
                             edges[q], edges[q + 1], epsabs=1e-13)[0] for q in range(4))
    assert abs(gaussian_msqe(levels) - ref) < 1e-10


def test_printed_codebook_is_near_optimal():
    c, _, mse_opt, _ = lloyd_max_gaussian([-1, -0.3, 0.3, 1], iters=5000)
    mse_printed = gaussian_msqe(CODEBOOK)
    assert mse_printed >= mse_opt
    assert mse_printed / mse_opt - 1.0 < 1e-3
