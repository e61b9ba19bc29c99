"""Plain, slow fp64 CPU oracle for block-wise low-bit weight quantization and
the products against the quantized weights.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The product (``bit_weight_quantized_qw_amd``) never imports it,
and the two share no code: no kernels, headers, helpers, tables or constant
generators. The oracle is written from the pages that define the method:

* "On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)" (otf-llm 4.0.1 package
  description): the adaptive non-uniform 2-bit code -- Lloyd-Max Gaussian
  codebook (section 2), per-group closed-form least squares scale and offset
  (section 3), four codes per byte ("Key v4.0 Innovations"), profile-guided
  FP16 outlier anchors (section 4).
* "AirQuant" README, "Fundamentacao Teorica e Arquitetura" item 2 and
  "Fontes": NF4 (NormalFloat4, QLoRA) block-wise weight quantization.
* the OTF-LLM page's "Comparative Analysis: INT4 (v3.2) vs INT2 Non-Uniform
  (v4.0)" and "Method Comparison Table": the v3.2 INT4 format (uniform
  symmetric grid, two codes per byte, a static channel permutation, the top
  1% channels in FP16).
* the gated activation between the gate/up and down projections of the
  decoder blocks the OTF-LLM page quantizes (``mlp``): the pages do not name
  it; the reading (SiLU, gate and up as one merged matrix) is stated there.

Where the pages leave a step open, the reading taken is stated in the
docstring of the function that takes it. Every function here is pinned by a
``-m "not gpu"`` test to something other than itself (textbook results,
closed forms, library routines, brute force, hand-derived bit patterns),
except the two marked "parity unpinned" below:

* ``claims.uniform_vs_lloyd_mse_ratio`` (the page's 4.2x MSE claim): parity
  unpinned -- the page gives no setting in which the ratio is reproduced.
* the GEMV/GEMM products have no worked example on the pages; they are pinned
  only through special cases (one-hot inputs, closed-form row sums, brute
  force on tiny shapes).
* ``nf4.NF4_DELTA`` (the outermost quantile probability of the NF4 levels):
  parity unpinned. The pages name NF4 and QLoRA but print no level, so the
  absolute values of the table rest on this reading of the construction;
  the tests pin only that the levels are the normal quantiles at evenly
  spaced probabilities from delta to 1/2 (the shape of the construction),
  not delta itself.
"""

from .codebook import CODEBOOK_F32, CODEBOOK, lloyd_max_gaussian, gaussian_msqe
from .rounding import fp16_rne, f32_to_bf16_rne_bits, bf16_bits_to_f64
from .quant2bit import (GROUP_2BIT, OLS_EPS, assign_codes_2bit, fit_2bit_groups, reassign_nearest_2bit, quantize_2bit,
                        pack_2bit, unpack_2bit, dequant_2bit, sz_interleaved)
from .nf4 import (BLOCK_NF4, nf4_levels, quantize_nf4, pack_nf4, unpack_nf4,
                  dequant_nf4)
from .outliers import (outlier_count, profile_abs_sum, profile_absmean, channel_scores,
                       select_outliers, SCORE_MEANABS, SCORE_L2)
from .int4perm import (GROUP_INT4, QMAX_INT4, ANCHOR_FRAC_INT4, int4_permutation, permute_cols,
                       quantize_int4, pack_int4, unpack_int4, dequant_int4, gemv_int4_ref,
                       prefill_weight_bf16_int4)
from .products import (gemv_2bit_ref, gemv_nf4_ref, prefill_weight_bf16_2bit,
                       prefill_weight_bf16_nf4, gemm_prefill_ref)
from .mlp import silu, swiglu_ref, gemv_2bit_swiglu_ref

__all__ = [
    "CODEBOOK_F32", "CODEBOOK", "lloyd_max_gaussian", "gaussian_msqe",
    "fp16_rne", "f32_to_bf16_rne_bits", "bf16_bits_to_f64",
    "GROUP_2BIT", "OLS_EPS", "assign_codes_2bit", "fit_2bit_groups", "reassign_nearest_2bit", "quantize_2bit", "pack_2bit", "sz_interleaved",
    "unpack_2bit", "dequant_2bit",
    "BLOCK_NF4", "nf4_levels", "quantize_nf4", "pack_nf4", "unpack_nf4",
    "dequant_nf4",
    "outlier_count", "profile_abs_sum", "profile_absmean", "channel_scores", "select_outliers",
    "SCORE_MEANABS", "SCORE_L2",
    "GROUP_INT4", "QMAX_INT4", "ANCHOR_FRAC_INT4", "int4_permutation", "permute_cols",
    "quantize_int4", "pack_int4", "unpack_int4", "dequant_int4", "gemv_int4_ref",
    "prefill_weight_bf16_int4",
    "gemv_2bit_ref", "gemv_nf4_ref", "prefill_weight_bf16_2bit",
    "prefill_weight_bf16_nf4", "gemm_prefill_ref",
    "silu", "swiglu_ref", "gemv_2bit_swiglu_ref",
]
