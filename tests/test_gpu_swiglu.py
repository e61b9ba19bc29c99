"""GPU parity of qgemv_2bit_swiglu (the merged gate/up GEMV with the gated
activation in its epilogue) with the fp64 oracle (oracle.gemv_2bit_swiglu_ref
on the oracle's own quantization of the merged matrix, anchors chosen by
oracle.select_outliers): fp32 output within the fp32 GEMV bound, fp16 output
equal to nearest-even of the fp32 output bit for bit, and the 32B block's
merged 55296 x 5120 gate/up matrix on sampled outputs."""

import numpy as np
import pytest

import oracle
from bit_weight_quantized_qw_amd import inputs, qw
from gpu_util import TOL, TOL_F32_GEMV, norm_err, to_dev, f16_dev

pytestmark = pytest.mark.gpu


def _pack(W, idx):
    idd = to_dev(np.asarray(idx, np.int32)) if idx is not None and len(idx) else None
    return qw.qw_pack(to_dev(W), qw.QW_FMT_2BIT_G32, idd)


def _ref(W, x16, idx):
    r = oracle.quantize_2bit(W, idx)
    return oracle.gemv_2bit_swiglu_ref(x16, r["q"], r["S"], r["Z"], r["idx"], r["W_O"])


def _run(pw, x16, f32):
    import torch
    y = qw.qgemv_2bit_swiglu(pw, f16_dev(x16), out_dtype=torch.float32 if f32 else torch.float16)
    return y.float().cpu().numpy()


# (I, K): one tile pair, several pairs with a ragged share per workgroup,
# an odd and an even workgroup count (the even one splits each CU's share of
# pairs between two workgroups, unevenly here: 600 pairs, 512 workgroups),
# the 32B block's hidden size
SHAPES = [(16, 512), (48, 1024), (272, 2048), (9600, 512), (1040, 5120)]


@pytest.mark.parametrize("I,K", SHAPES)
@pytest.mark.parametrize("B", [1, 2, 3, 8])
@pytest.mark.parametrize("frac", [0.0, 0.035])
def test_swiglu_small(I, K, B, frac):
    W = inputs.weight(2 * I, K, workload=91)
    X = inputs.profile(64, K, workload=91)
    idx = oracle.select_outliers(W, X, frac) if frac else None
    x = inputs.act_f16(B, K, workload=91)
    pw = _pack(W, idx)
    ref = _ref(W, x, idx)
    y32 = _run(pw, x, True)
    y16 = _run(pw, x, False)
    assert y32.shape == (B, I)
    e = norm_err(y32, ref)
    print(f"I={I} K={K} B={B} anchors={0 if idx is None else len(idx)}: fp32-out err {e:.3e}")
    assert e <= TOL_F32_GEMV
    np.testing.assert_array_equal(y16.astype(np.float16), y32.astype(np.float16))


def test_swiglu_zero_input_gives_zero():
    W = inputs.weight(96, 1024, workload=92)
    pw = _pack(W, None)
    y = _run(pw, np.zeros((2, 1024), np.float16), True)
    assert not np.any(y)


def test_swiglu_32b_block_sampled():
    """The 32B block's gate and up projections as one 55296 x 5120 matrix
    with 3.5% anchors: the device's anchor choice equals the oracle's over
    the merged matrix, and 384 sampled outputs (both halves of each) match."""
    import torch
    I, K = 27648, 5120
    W = inputs.weight(2 * I, K, workload=93)
    X = inputs.profile(256, K, workload=93)
    idx = oracle.select_outliers(W, X, 0.035)
    dev_idx = qw.qw_select_outliers(to_dev(W), to_dev(X), 0.035)
    np.testing.assert_array_equal(np.sort(dev_idx.cpu().numpy()), np.sort(idx))
    pw = _pack(W, idx)
    x = inputs.act_f16(4, K, workload=93)
    y = _run(pw, x, True)
    torch.cuda.synchronize()
    ns = np.sort(np.random.default_rng(93).choice(I, 384, replace=False))
    rows = np.concatenate([ns, I + ns])
    ref = _ref(W[rows], x, idx)
    e = norm_err(y[:, ns], ref)
    print(f"55296x5120 anchors={len(idx)} B=4 sampled err {e:.3e}")
    assert e <= TOL_F32_GEMV


def test_swiglu_rejects_bad_shapes():
    import torch
    W = inputs.weight(48, 512, workload=94)  # N = 48: not two halves of whole tiles
    pw = _pack(W, None)
    x = torch.zeros((1, 512), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        qw.qgemv_2bit_swiglu(pw, x)
    v = pw.view()
    y = torch.zeros(64, dtype=torch.float16, device="cuda")
    import ctypes
    st = qw.lib().qgemv_2bit_swiglu(ctypes.byref(v), qw._ptr(x), 1, qw._ptr(y), qw.QW_DT_F16, qw._stream())
    assert st == qw.QW_ERR_INVALID_ARG
    W2 = inputs.weight(64, 96, workload=94)  # K % 512 != 0
    pw2 = _pack(W2, None)
    x2 = torch.zeros((1, 96), dtype=torch.float16, device="cuda")
    with pytest.raises(qw.QwError) as e:
        qw.qgemv_2bit_swiglu(pw2, x2)
    assert e.value.status == qw.QW_ERR_UNSUPPORTED
