"""The pages' quantitative claims around the method.

* section 1 bandwidth argument: decode speed bounded by bus bandwidth over
  the weight bytes read per token -- closed-form arithmetic on the printed
  figures;
* section 2 "4.2x lower MSE": parity unpinned. Measured here on Gaussian
  groups and reported; only the qualitative direction (the non-uniform code
  beats the min-max uniform grid) is asserted.
"""

import json
import os

import numpy as np

from oracle.claims import uniform_vs_lloyd_mse_ratio
from bit_weight_quantized_qw_amd import inputs


def _g(golden_dir):
    with open(os.path.join(golden_dir, "pages_figures.json")) as f:
        return json.load(f)


def test_bandwidth_argument_arithmetic(golden_dir):
    b = _g(golden_dir)["bandwidth_argument"]
    fp16 = b["bus_gb_per_s"] / b["fp16_gb_per_token"]
    two = b["bus_gb_per_s"] / b["twobit_gb_per_token"]
    assert abs(fp16 - b["fp16_tokens_per_s_approx"]) / b["fp16_tokens_per_s_approx"] < 0.05
    assert two >= b["twobit_tokens_per_s_at_least"]


def test_two_bit_bytes_per_weight():
    # 2-bit codes + one fp16 pair per 32 weights = 3 bits per weight
    assert (2 * 32 + 2 * 16) / 32 == 3.0


def test_mse_ratio_direction_only(golden_dir):
    W = inputs.weight(256, 1024, workload=51)
    ratio = uniform_vs_lloyd_mse_ratio(W)
    claim = _g(golden_dir)["mse_ratio_claim"]["value"]
    print(f"uniform/min-max vs Lloyd+OLS MSE ratio on N(0,0.02^2) groups of 32: "
          f"{ratio:.3f} (page claims {claim})")
    assert ratio > 1.0
