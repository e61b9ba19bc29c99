"""GPU parity of the prefill GEMM (qgemm_prefill) with the fp64 oracle that
models the bf16 dequantized weights: fp32 output within 1e-3 normwise, and
bf16 output equal to nearest-even of the fp32 output bit for bit. The
70B-shaped workload (2048 x 8192 times 28672 x 8192) is checked on sampled
outputs."""

import numpy as np
import pytest

import oracle
from bit_weight_quantized_qw_amd import inputs, qw
from gpu_util import TOL, norm_err, to_dev, bf16_dev

pytestmark = pytest.mark.gpu


def _pack(W, fmt, idx=None):
    idd = to_dev(np.asarray(idx, np.int32)) if idx is not None and len(idx) else None
    return qw.qw_pack(to_dev(W), fmt, idd)


def _wbits(W, fmt, idx=None):
    if fmt == qw.QW_FMT_2BIT_G32:
        r = oracle.quantize_2bit(W, idx)
        return oracle.prefill_weight_bf16_2bit(r["q"], r["S"], r["Z"], r["idx"], r["W_O"])
    q, a = oracle.quantize_nf4(W)
    return oracle.prefill_weight_bf16_nf4(q, a)


def _run(pw, Xbits, f32=True):
    import torch
    Y = qw.qgemm_prefill(pw, bf16_dev(Xbits), out_dtype=torch.float32 if f32 else torch.bfloat16)
    return Y


FMTS = [qw.QW_FMT_2BIT_G32, qw.QW_FMT_NF4_B64]


SMALL = [(300, 200, 512), (1, 1, 64), (257, 129, 128), (512, 1024, 2048), (513, 300, 192), (64, 777, 64)]


# wide=None: the library's own split between 256- and 128-wide column tiles;
# "0": 128-wide tiles only; "1": one 256-wide column tile, the rest 128-wide
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", SMALL)
@pytest.mark.parametrize("wide", [None, "0", "1"])
def test_prefill_small(fmt, M, N, K, wide, tune):
    import torch
    if wide is not None:
        tune(qw.QW_TUNE_PREFILL_WIDE_TILES, int(wide))
    W = inputs.weight(N, K, workload=80)
    X = inputs.act_bf16_bits(M, K, workload=80)
    pw = _pack(W, fmt)
    Y32 = _run(pw, X)
    ref = oracle.gemm_prefill_ref(X, _wbits(W, fmt))
    e = norm_err(Y32.cpu().numpy(), ref)
    print(f"fmt={fmt} {M}x{N}x{K}: err {e:.3e}")
    assert e <= TOL
    Yb = _run(pw, X, f32=False)
    np.testing.assert_array_equal(Yb.view(torch.int16).cpu().numpy(),
                                  Y32.to(torch.bfloat16).view(torch.int16).cpu().numpy())


def test_prefill_2bit_with_anchors():
    W = inputs.weight(96, 256, workload=81)
    idx = np.array([0, 1, 31, 32, 63, 64, 200, 255], np.int32)
    X = inputs.act_bf16_bits(70, 256, workload=81)
    pw = _pack(W, qw.QW_FMT_2BIT_G32, idx)
    ref = oracle.gemm_prefill_ref(X, _wbits(W, qw.QW_FMT_2BIT_G32, idx))
    assert norm_err(_run(pw, X).cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("fmt", FMTS)
def test_prefill_70b_shape_sampled(fmt):
    M, N, K = 2048, 28672, 8192
    W = inputs.weight(N, K, workload=5)
    X = inputs.act_bf16_bits(M, K, workload=5)
    pw = _pack(W, fmt)
    Y = _run(pw, X).cpu().numpy()
    g = np.random.default_rng(5)
    ms = np.sort(g.choice(M, 48, replace=False))
    ns = np.sort(g.choice(N, 320, replace=False))
    ref = oracle.gemm_prefill_ref(X[ms], _wbits(W[ns], fmt))
    e = norm_err(Y[np.ix_(ms, ns)], ref)
    print(f"70B-shaped prefill fmt={fmt}: sampled err {e:.3e}")
    assert e <= TOL
