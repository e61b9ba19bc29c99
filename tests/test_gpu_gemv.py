"""GPU parity of the decode GEMVs (qgemv_2bit, qgemv_nf4, qgemv_2bit_grouped)
with the fp64 oracle: normwise relative error <= 1e-3 (fp32 accumulation,
fp16 output), fp16 output == nearest-even of the fp32 output, and exact
zeros for a zero input."""

import numpy as np
import pytest

import oracle
from bit_weight_quantized_qw_amd import inputs, qw
from gpu_util import TOL, TOL_F32_GEMV, norm_err, to_dev, f16_dev, oracle_2bit, oracle_nf4

pytestmark = pytest.mark.gpu


def _packed_2bit(W, idx=None):
    idd = to_dev(np.asarray(idx, np.int32)) if idx is not None and len(idx) else None
    return qw.qw_pack(to_dev(W), qw.QW_FMT_2BIT_G32, idd)


def _run_2bit(pw, x16, f32=False):
    import torch
    y = qw.qgemv_2bit(pw, f16_dev(x16), out_dtype=torch.float32 if f32 else torch.float16)
    return y.float().cpu().numpy()


def _ref_2bit(W, x16, idx=None):
    r = oracle.quantize_2bit(W, idx)
    return oracle.gemv_2bit_ref(x16, r["q"], r["S"], r["Z"], r["idx"], r["W_O"])


def test_gemv_2bit_single_layer_2048():
    W = inputs.weight(2048, 2048, workload=1)
    x = inputs.act_f16(1, 2048, workload=1)
    pw = _packed_2bit(W)
    ref = _ref_2bit(W, x)
    y16 = _run_2bit(pw, x)
    y32 = _run_2bit(pw, x, f32=True)
    e = norm_err(y32, ref)
    print(f"2048x2048 B=1 fp32-out err {e:.3e}, fp16-out err {norm_err(y16, ref):.3e}")
    assert e <= TOL_F32_GEMV and norm_err(y16, ref) <= TOL
    np.testing.assert_array_equal(y16.astype(np.float16), y32.astype(np.float16))


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 6, 7, 8])
def test_gemv_2bit_14b_shape_with_anchors(B):
    W = inputs.weight(13824, 5120, workload=3)
    X = inputs.profile(256, 5120, workload=3)
    idx = oracle.select_outliers(W, X, 0.035)
    x = inputs.act_f16(B, 5120, workload=3)
    pw = _packed_2bit(W, idx)
    y = _run_2bit(pw, x)
    e = norm_err(y, _ref_2bit(W, x, idx))
    print(f"13824x5120 anchors=179 B={B} err {e:.3e}")
    assert e <= TOL


@pytest.mark.parametrize("B", [5, 8])
def test_gemv_2bit_wide_batch_rows_equal_single_rows(B, tune):
    """A batch that fits one matrix-core pass only without the raw x copy in
    LDS (anchors then gathered from global x) gives every row the bits of
    that row computed alone."""
    W = inputs.weight(4096, 5120, workload=81)
    X = inputs.profile(64, 5120, workload=81)
    idx = oracle.select_outliers(W, X, 0.035)
    x = inputs.act_f16(B, 5120, workload=81)
    pw = _packed_2bit(W, idx)
    tune(qw.QW_TUNE_GEMV2_PATH, 0)
    yB = _run_2bit(pw, x, f32=True)
    for b in range(B):
        np.testing.assert_array_equal(yB[b], _run_2bit(pw, x[b:b + 1], f32=True)[0], err_msg=f"row {b}")
    assert norm_err(yB, _ref_2bit(W, x, idx)) <= TOL


@pytest.mark.parametrize("N,K,n_anchor", [(1, 32, 0), (7, 96, 2), (33, 1056, 5), (130, 2080, 0),
                                          (64, 3072, 40), (5, 27648, 967), (300, 27648, 967)])
@pytest.mark.parametrize("B", [1, 2, 4])
def test_gemv_2bit_ragged(N, K, n_anchor, B):
    W = inputs.weight(N, K, workload=70)
    idx = np.sort(np.random.default_rng(N * K).choice(K, n_anchor, replace=False)).astype(np.int32)
    x = inputs.act_f16(B, K, workload=70)
    pw = _packed_2bit(W, idx if n_anchor else None)
    e = norm_err(_run_2bit(pw, x, f32=True), _ref_2bit(W, x, idx if n_anchor else None))
    assert e <= TOL, e


def test_gemv_2bit_zero_input_gives_zero():
    W = inputs.weight(64, 512, workload=71)
    pw = _packed_2bit(W, np.array([3, 300], np.int32))
    y = _run_2bit(pw, np.zeros((2, 512), np.float16), f32=True)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("scale", [1e-4, 1.0, 300.0, 3000.0, 60000.0])
def test_gemv_2bit_input_scales(scale):
    W = inputs.weight(256, 1024, workload=72)
    x = (inputs.act_f16(2, 1024, workload=72).astype(np.float32) * scale)
    x = np.clip(x, -65504, 65504).astype(np.float16)
    pw = _packed_2bit(W)
    e = norm_err(_run_2bit(pw, x, f32=True), _ref_2bit(W, x))
    print(f"input scale {scale}: err {e:.3e}")
    assert e <= TOL


def test_gemv_2bit_one_hot_reads_columns():
    W = inputs.weight(96, 256, workload=73)
    idx = np.array([5, 200], np.int32)
    pw = _packed_2bit(W, idx)
    r = oracle.quantize_2bit(W, idx)
    Wh = oracle.dequant_2bit(r["q"], r["S"], r["Z"])
    for k in (0, 5, 17, 31, 32, 200, 255):
        x = np.zeros((1, 256), np.float16)
        x[0, k] = 1
        y = _run_2bit(pw, x, f32=True)[0]
        ref = r["W_O"][:, list(idx).index(k)].astype(np.float64) if k in idx else Wh[:, k]
        assert norm_err(y, ref) <= 1e-6


def test_gemv_2bit_grouped_equals_separate():
    import torch
    K = 5120
    pws, xs = [], inputs.act_f16(1, K, workload=74)
    for p, N in enumerate((5120, 1024, 1024)):
        W = inputs.weight(N, K, workload=74, proj=p)
        X = inputs.profile(64, K, workload=74, proj=p)
        pws.append(_packed_2bit(W, oracle.select_outliers(W, X, 0.035)))
    xd = f16_dev(xs)
    ys = qw.qgemv_2bit_grouped(pws, xd, out_dtype=torch.float32)
    for pw, yg in zip(pws, ys):
        ysep = qw.qgemv_2bit(pw, xd, out_dtype=torch.float32)
        np.testing.assert_array_equal(yg.cpu().numpy(), ysep.cpu().numpy())


def _run_nf4(W, x16, f32=False):
    import torch
    pw = qw.qw_pack(to_dev(W), qw.QW_FMT_NF4_B64)
    y = qw.qgemv_nf4(pw, f16_dev(x16), out_dtype=torch.float32 if f32 else torch.float16)
    return y.float().cpu().numpy()


@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_gemv_nf4_llama7b_mlp_shape(B):
    W = inputs.weight(11008, 4096, workload=2)
    x = inputs.act_f16(B, 4096, workload=2)
    q, a = oracle.quantize_nf4(W)
    ref = oracle.gemv_nf4_ref(x, q, a)
    e = norm_err(_run_nf4(W, x, f32=True), ref)
    e16 = norm_err(_run_nf4(W, x), ref)
    print(f"NF4 11008x4096 B={B} err {e:.3e} (fp16 out {e16:.3e})")
    assert e <= TOL_F32_GEMV and e16 <= TOL


def test_gemv_2bit_llama7b_mlp_shape():
    W = inputs.weight(11008, 4096, workload=2)
    x = inputs.act_f16(1, 4096, workload=2)
    pw = _packed_2bit(W)
    e = norm_err(_run_2bit(pw, x), _ref_2bit(W, x))
    assert e <= TOL


@pytest.mark.parametrize("N,K", [(3, 64), (5, 192), (64, 4160), (9, 28672)])
@pytest.mark.parametrize("B", [1, 3])
def test_gemv_nf4_ragged(N, K, B):
    W = inputs.weight(N, K, workload=75)
    W[0, :64] = 0.0
    x = inputs.act_f16(B, K, workload=75)
    q, a = oracle.quantize_nf4(W)
    e = norm_err(_run_nf4(W, x, f32=True), oracle.gemv_nf4_ref(x, q, a))
    assert e <= TOL_F32_GEMV, e


@pytest.mark.parametrize("scale", [1e-4, 1.0, 300.0, 60000.0])
def test_gemv_nf4_input_scales(scale):
    """fp16 activations from subnormal to near-overflow magnitudes."""
    W = inputs.weight(256, 1024, workload=77)
    x = (inputs.act_f16(2, 1024, workload=77).astype(np.float32) * scale)
    x = np.clip(x, -65504, 65504).astype(np.float16)
    q, a = oracle.quantize_nf4(W)
    e = norm_err(_run_nf4(W, x, f32=True), oracle.gemv_nf4_ref(x, q, a))
    print(f"NF4 input scale {scale}: err {e:.3e}")
    assert e <= TOL


def test_gemv_nf4_one_hot_reads_columns():
    """x = e_k gives fl32(absmax * L[q]) of column k: one product, one rounding."""
    W = inputs.weight(200, 512, workload=78)
    q, a = oracle.quantize_nf4(W)
    x = np.zeros((2, 512), np.float16)
    x[0, 7] = 1.0
    x[1, 300] = 1.0
    y = _run_nf4(W, x, f32=True)
    L = oracle.nf4_levels().astype(np.float64)
    np.testing.assert_array_equal(y[0], (a[:, 7 // 64].astype(np.float64) * L[q[:, 7]]).astype(np.float32))
    np.testing.assert_array_equal(y[1], (a[:, 300 // 64].astype(np.float64) * L[q[:, 300]]).astype(np.float32))


@pytest.mark.parametrize("B", [5, 6, 7])
def test_gemv_nf4_batch_slices(B):
    """Batches cut into 4/2/1-row launches: every row as the oracle."""
    W = inputs.weight(1000, 4096, workload=79)
    x = inputs.act_f16(B, 4096, workload=79)
    q, a = oracle.quantize_nf4(W)
    e = norm_err(_run_nf4(W, x, f32=True), oracle.gemv_nf4_ref(x, q, a))
    assert e <= TOL, e


def test_gemv_nf4_fp16_out_is_rounded_fp32_out():
    W = inputs.weight(512, 1024, workload=76)
    x = inputs.act_f16(2, 1024, workload=76)
    np.testing.assert_array_equal(_run_nf4(W, x).astype(np.float16),
                                  _run_nf4(W, x, f32=True).astype(np.float16))


def test_timed_call_records_kernel_duration_and_same_result():
    import torch
    W = inputs.weight(4096, 4096, workload=77)
    x = f16_dev(inputs.act_f16(1, 4096, workload=77))
    pw = _packed_2bit(W)
    y0 = qw.qgemv_2bit(pw, x, out_dtype=torch.float32)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qw.qw_time_next_call(s, e)
    y1 = qw.qgemv_2bit(pw, x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    print(f"timed qgemv_2bit 4096x4096: {ms * 1e3:.2f} us")
    assert 0.0 < ms < 50.0
    assert torch.equal(y0, y1)
    # the pair was consumed: a second call does not re-record it
    qw.qgemv_2bit(pw, x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert s.elapsed_time(e) == ms


@pytest.mark.parametrize("N,K,n_anchor,B", [(2048, 2048, 0, 1), (13824, 5120, 179, 1), (1000, 5120, 179, 3),
                                            (64, 3072, 40, 2), (300, 27648, 967, 1), (777, 4096, 0, 8),
                                            (16, 512, 5, 6), (17, 1024, 3, 7)])
def test_gemv_2bit_matrix_core_and_vector_paths(N, K, n_anchor, B, tune):
    """Both kernels of qgemv_2bit (matrix-core path for K % 512 == 0 when
    the shape fits it, vector-ALU path otherwise or when forced) against the
    oracle on the same inputs."""
    W = inputs.weight(N, K, workload=78)
    rng = np.random.default_rng(N + K)
    idx = np.sort(rng.choice(K, n_anchor, replace=False)).astype(np.int32) if n_anchor else None
    x = inputs.act_f16(B, K, workload=78)
    pw = _packed_2bit(W, idx)
    ref = _ref_2bit(W, x, idx)
    tune(qw.QW_TUNE_GEMV2_PATH, 0)
    y_mc = _run_2bit(pw, x, f32=True)
    tune(qw.QW_TUNE_GEMV2_PATH, 1)
    y_va = _run_2bit(pw, x, f32=True)
    e_mc, e_va = norm_err(y_mc, ref), norm_err(y_va, ref)
    print(f"{N}x{K} anchors={n_anchor} B={B}: matrix-core err {e_mc:.3e}, vector err {e_va:.3e}")
    assert e_mc <= TOL_F32_GEMV and e_va <= TOL_F32_GEMV


def test_gemv_2bit_largest_k_each_path(tune):
    """The largest rows each kernel takes whole at batch 1: K = 40960 on the
    matrix cores (its x limbs and 1433 anchor slots fill most of the LDS, the
    anchors gathered from global x) and K = 32736 on the vector ALUs (the
    prepared x takes 5 K bytes of the 160 KB); both against the oracle with
    3.5% anchors. At K = 40960 batch 2 needs K parts: through a workspace it
    runs, without one it is refused."""
    import torch
    for K, path in ((40960, 0), (32736, 1)):
        W = inputs.weight(48, K, workload=85)
        X = inputs.profile(32, K, workload=85)
        idx = oracle.select_outliers(W, X, 0.035)
        x = inputs.act_f16(2, K, workload=85)
        pw = _packed_2bit(W, idx)
        tune(qw.QW_TUNE_GEMV2_PATH, path)
        y = _run_2bit(pw, x[:1], f32=True)
        e = norm_err(y, _ref_2bit(W, x[:1], idx))
        print(f"48x{K} anchors={len(idx)} path={path}: err {e:.3e}")
        assert e <= TOL_F32_GEMV
        if K == 40960:
            ws = qw.gemv_workspace(pw, 2)
            assert ws is not None
            y2 = qw.qgemv_2bit_ws(pw, f16_dev(x), ws, out_dtype=torch.float32).cpu().numpy()
            assert norm_err(y2, _ref_2bit(W, x, idx)) <= TOL_F32_GEMV
            with pytest.raises(qw.QwError) as ex:
                qw.qgemv_2bit(pw, f16_dev(x))
            assert ex.value.status == qw.QW_ERR_UNSUPPORTED


def test_gemv_2bit_half_the_channels_anchored():
    """A degenerate anchor set: half of the channels (every second one,
    including the first and the last group's edges) kept in fp16."""
    K = 1024
    W = inputs.weight(40, K, workload=86)
    idx = np.arange(1, K, 2, dtype=np.int32)
    idx[0] = 0
    x = inputs.act_f16(3, K, workload=86)
    pw = _packed_2bit(W, idx)
    e = norm_err(_run_2bit(pw, x, f32=True), _ref_2bit(W, x, idx))
    print(f"40x{K} with {len(idx)} anchors: err {e:.3e}")
    assert e <= TOL_F32_GEMV


@pytest.mark.parametrize("N,K,n_anchor,B", [(1024, 5120, 179, 1), (2048, 2048, 0, 1), (11008, 4096, 0, 1),
                                            (1000, 5120, 179, 3), (64, 3072, 40, 2)])
def test_gemv_2bit_ring_depth_same_bits(N, K, n_anchor, B, tune):
    """The matrix-core kernel's two ring depths (prefetch slots per wave)
    change only when loads are issued, never the arithmetic: same bits."""
    W = inputs.weight(N, K, workload=79)
    rng = np.random.default_rng(N * 7 + K)
    idx = np.sort(rng.choice(K, n_anchor, replace=False)).astype(np.int32) if n_anchor else None
    x = inputs.act_f16(B, K, workload=79)
    pw = _packed_2bit(W, idx)
    tune(qw.QW_TUNE_GEMV2_PATH, 0)
    tune(qw.QW_TUNE_GEMV2_DEEP_RING, 0)
    y3 = _run_2bit(pw, x, f32=True)
    tune(qw.QW_TUNE_GEMV2_DEEP_RING, 1)
    y6 = _run_2bit(pw, x, f32=True)
    ref = _ref_2bit(W, x, idx)
    print(f"{N}x{K} anchors={n_anchor} B={B}: shallow err {norm_err(y3, ref):.3e} deep err {norm_err(y6, ref):.3e} "
          f"max |diff| {np.abs(y3 - y6).max():.3e}")
    np.testing.assert_array_equal(y3, y6)


@pytest.mark.parametrize("N,K,B", [(11008, 4096, 1), (4096, 11008, 1), (300, 27648, 2), (1000, 4096, 4), (77, 640, 1)])
def test_gemv_nf4_ring_depth_same_bits(N, K, B, tune):
    """NF4 GEMV with 3 and 6 row slots per wave: same bits, and within the
    tolerance of the oracle."""
    W = inputs.weight(N, K, workload=82)
    x = inputs.act_f16(B, K, workload=82)
    q, a = oracle.quantize_nf4(W)
    tune(qw.QW_TUNE_NF4_DEEP_RING, 0)
    y3 = _run_nf4(W, x, f32=True)
    tune(qw.QW_TUNE_NF4_DEEP_RING, 1)
    y6 = _run_nf4(W, x, f32=True)
    e = norm_err(y3, oracle.gemv_nf4_ref(x, q, a))
    print(f"NF4 {N}x{K} B={B}: err {e:.3e} max |diff| {np.abs(y3 - y6).max():.3e}")
    assert e <= TOL
    np.testing.assert_array_equal(y3, y6)
