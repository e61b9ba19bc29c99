"""GPU parity of the v3.2 INT4 permutation format (the OTF-LLM page's
"Comparative Analysis" and "Method Comparison Table") with the fp64 oracle:
the channel permutation and the packed codes, scales and fp16 anchors
bit-exact; the permuted-order gather bit-exact; the decode GEMV (batches
1-8) and the prefill GEMM within 1e-3 normwise, fp16/bf16 outputs equal to
nearest-even of the fp32 outputs bit for bit. Shapes span several row and
K tiles with ragged tails, no anchors and up to 1% anchors, the 14B-shaped
13824x5120 decode and a 70B-shaped 8192x28672 matrix at full size."""

import numpy as np
import pytest

import oracle
from bit_weight_quantized_qw_amd import inputs, qw
from gpu_util import TOL, TOL_F32_GEMV, norm_err, to_dev, f16_dev, bf16_dev, assert_bits_equal

pytestmark = pytest.mark.gpu


def _perm(W, Xp):
    return oracle.int4_permutation(W, Xp)


def _pack(W, perm, n_out):
    return qw.qw_pack_int4(to_dev(W), to_dev(np.asarray(perm, np.int32)), n_out)


def _check_pack(pw, r):
    assert_bits_equal(pw.host_codes(), oracle.pack_int4(r["q"]), "int4 codes")
    assert_bits_equal(pw.host_scales(), r["s"], "int4 scales")
    if r["W_O"].shape[1]:
        assert_bits_equal(pw.host_out_w()[:, :r["W_O"].shape[1]], r["W_O"], "int4 anchors")
        assert np.all(pw.host_out_w()[:, r["W_O"].shape[1]:] == 0)


@pytest.mark.parametrize("N,K,n_out", [(200, 3072, 30), (77, 1024, 0), (1, 32, 0), (33, 160, 1),
                                       (5, 4096, 40)])
def test_pack_and_permutation_bit_exact(N, K, n_out):
    W = inputs.weight(N, K, workload=110)
    Xp = inputs.profile(64, K, workload=110)
    perm = _perm(W, Xp)
    got = qw.qw_select_perm(to_dev(W), to_dev(Xp)).cpu().numpy()
    np.testing.assert_array_equal(got, perm)
    r = oracle.quantize_int4(W, perm, n_out)
    _check_pack(_pack(W, perm, n_out), r)


@pytest.mark.parametrize("kind", ["zero", "const", "alternating", "ramp"])
def test_pack_structured_weights(kind):
    N, K = 24, 256
    W = inputs.special_weight(kind, N, K, workload=111)
    perm = np.random.default_rng(111).permutation(K).astype(np.int32)
    r = oracle.quantize_int4(W, perm, 3)
    _check_pack(_pack(W, perm, 3), r)


def test_pack_from_fp16_and_bf16_weights():
    import torch
    N, K = 64, 512
    W = inputs.weight(N, K, workload=112)
    perm = np.random.default_rng(112).permutation(K).astype(np.int32)
    for dt in (torch.float16, torch.bfloat16):
        Wt = torch.from_numpy(W).to(dt)
        r = oracle.quantize_int4(Wt.float().numpy(), perm, 5)
        pw = qw.qw_pack_int4(Wt.cuda(), to_dev(perm), 5)
        _check_pack(pw, r)


def test_permute_cols_all_dtypes():
    import torch
    M, K = 37, 1056
    perm = np.random.default_rng(113).permutation(K).astype(np.int32)
    X = inputs.profile(M, K, workload=113)
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        Xt = torch.from_numpy(X).to(dt).cuda()
        got = qw.qw_permute_cols(Xt, to_dev(perm))
        torch.cuda.synchronize()
        assert torch.equal(got, Xt[:, torch.from_numpy(perm.astype(np.int64)).cuda()]), dt


def _gemv(pw, x_p16, f32=True):
    import torch
    y = qw.qgemv_int4(pw, f16_dev(x_p16), out_dtype=torch.float32 if f32 else torch.float16)
    return y.float().cpu().numpy()


# K a multiple of 512 runs on the matrix cores (one super-chunk, one row,
# a ragged tile, anchors ending inside and at the edge of a group), the
# others on the vector ALUs
@pytest.mark.parametrize("N,K,n_out", [(200, 3072, 30), (77, 1024, 0), (1, 32, 0), (33, 160, 1),
                                       (300, 8192, 81), (50, 16384, 163), (1, 512, 0), (17, 512, 5),
                                       (16, 1536, 32)])
@pytest.mark.parametrize("B", [1, 2, 3, 5, 8])
def test_gemv_small(N, K, n_out, B):
    W = inputs.weight(N, K, workload=114)
    perm = np.random.default_rng(N + K).permutation(K).astype(np.int32)
    r = oracle.quantize_int4(W, perm, n_out)
    pw = _pack(W, perm, n_out)
    x_p = oracle.permute_cols(inputs.act_f16(B, K, workload=114), perm)
    ref = oracle.gemv_int4_ref(x_p, r["q"], r["s"], r["W_O"])
    y32 = _gemv(pw, x_p)
    y16 = _gemv(pw, x_p, f32=False)
    e = norm_err(y32, ref)
    print(f"int4 {N}x{K} anchors={n_out} B={B}: err {e:.3e}")
    assert e <= TOL_F32_GEMV
    np.testing.assert_array_equal(y16.astype(np.float16), y32.astype(np.float16))


# (N, K, n_out, B): batches the matrix-core kernel takes in one pass (with
# and without the raw x copy) and in slices (8 rows of K = 8192 as 3 + 3 + 2)
@pytest.mark.parametrize("N,K,n_out,B", [(200, 3072, 30, 1), (200, 3072, 30, 8), (300, 8192, 81, 3),
                                         (300, 8192, 81, 8), (50, 16384, 163, 1), (64, 5120, 51, 8)])
def test_gemv_both_kernels(N, K, n_out, B, tune):
    """Shapes the matrix-core kernel takes, run on it and, forced, on the
    vector-ALU kernel: both within the fp32 bound of the oracle. Their low
    bits differ (the two sum in different orders), which shows that the two
    calls ran different kernels."""
    W = inputs.weight(N, K, workload=117)
    perm = np.random.default_rng(N * K).permutation(K).astype(np.int32)
    r = oracle.quantize_int4(W, perm, n_out)
    pw = _pack(W, perm, n_out)
    x_p = oracle.permute_cols(inputs.act_f16(B, K, workload=117), perm)
    ref = oracle.gemv_int4_ref(x_p, r["q"], r["s"], r["W_O"])
    ys = []
    for path in (0, 1):
        tune(qw.QW_TUNE_INT4_PATH, path)
        y = _gemv(pw, x_p)
        e = norm_err(y, ref)
        print(f"int4 {N}x{K} anchors={n_out} B={B} path={path}: err {e:.3e}")
        assert e <= TOL_F32_GEMV
        ys.append(y)
    assert not np.array_equal(ys[0], ys[1])


def test_gemv_largest_k(tune):
    """The largest rows the matrix-core kernel takes whole at batch 1:
    K = 28672 with the raw x copy in LDS and K = 40960 without it (anchors
    gathered from global x), 1% anchors (287 and 409: several gather
    chunks); batch 2 at K = 40960 does not fit it and runs on the
    vector-ALU kernel. All against the oracle."""
    for K in (28672, 40960):
        N = 48
        W = inputs.weight(N, K, workload=116)
        perm = np.random.default_rng(K).permutation(K).astype(np.int32)
        n_out = oracle.outlier_count(K, 0.01)
        r = oracle.quantize_int4(W, perm, n_out)
        pw = _pack(W, perm, n_out)
        x_p = oracle.permute_cols(inputs.act_f16(2, K, workload=116), perm)
        for B in (1, 2):
            e = norm_err(_gemv(pw, x_p[:B]), oracle.gemv_int4_ref(x_p[:B], r["q"], r["s"], r["W_O"]))
            print(f"int4 {N}x{K} anchors={n_out} B={B}: err {e:.3e}")
            assert e <= TOL_F32_GEMV


def test_gemv_one_hot_and_zero_inputs():
    N, K, n_out = 40, 2048, 20
    W = inputs.weight(N, K, workload=115)
    perm = np.random.default_rng(115).permutation(K).astype(np.int32)
    r = oracle.quantize_int4(W, perm, n_out)
    pw = _pack(W, perm, n_out)
    cols = [0, 5, 19, 20, 31, 32, 1023, 2047]
    x = np.zeros((len(cols), K), np.float16)
    for b, j in enumerate(cols):
        x[b, j] = 1
    y = _gemv(pw, x)
    for b, j in enumerate(cols):
        want = r["W_O"][:, j].astype(np.float64) if j < n_out else \
            r["s"][:, j // 32].astype(np.float64) * r["q"][:, j]
        np.testing.assert_array_equal(y[b], want)
    assert np.all(_gemv(pw, np.zeros((3, K), np.float16)) == 0)


@pytest.mark.parametrize("B", [1, 4, 8])
def test_gemv_14b_shape(B):
    """13824x5120 with the top 1% (51) channels as anchors, permutation from
    a spiked calibration profile (the 14B decode shape)."""
    N, K = 13824, 5120
    W = inputs.weight(N, K, workload=3)
    Xp = inputs.profile(256, K, workload=3)
    perm = _perm(W, Xp)
    n_out = oracle.outlier_count(K, 0.01)
    assert n_out == 51
    r = oracle.quantize_int4(W, perm, n_out)
    pw = _pack(W, perm, n_out)
    _check_pack(pw, r)
    x_p = oracle.permute_cols(inputs.act_f16(B, K, workload=3), perm)
    e = norm_err(_gemv(pw, x_p), oracle.gemv_int4_ref(x_p, r["q"], r["s"], r["W_O"]))
    print(f"int4 13824x5120 B={B}: err {e:.3e}")
    assert e <= TOL_F32_GEMV


def test_gemv_70b_down_shape_sampled():
    """8192x28672 (286 anchors) at batch 1 and 3: all outputs against the
    oracle on 256 sampled rows; the device permutation equals the oracle's."""
    N, K = 8192, 28672
    W = inputs.weight(N, K, workload=6)
    Xp = inputs.profile(256, K, workload=6)
    perm = _perm(W, Xp)
    np.testing.assert_array_equal(qw.qw_select_perm(to_dev(W), to_dev(Xp)).cpu().numpy(), perm)
    n_out = oracle.outlier_count(K, 0.01)
    pw = _pack(W, perm, n_out)
    rows = np.sort(inputs.rng(6, 0, 0, 5).choice(N, 256, replace=False))
    r = oracle.quantize_int4(W[rows], perm, n_out)
    assert_bits_equal(pw.host_codes()[rows], oracle.pack_int4(r["q"]), "sampled codes")
    for B in (1, 3):
        x_p = oracle.permute_cols(inputs.act_f16(B, K, workload=6), perm)
        y = _gemv(pw, x_p)
        e = norm_err(y[:, rows], oracle.gemv_int4_ref(x_p, r["q"], r["s"], r["W_O"]))
        print(f"int4 8192x28672 B={B}: sampled err {e:.3e}")
        assert e <= TOL


def _prefill(pw, Xbits, f32=True):
    import torch
    return qw.qgemm_prefill(pw, bf16_dev(Xbits), out_dtype=torch.float32 if f32 else torch.bfloat16)


@pytest.mark.parametrize("M,N,K,n_out", [(300, 200, 512, 0), (257, 129, 128, 0), (512, 1024, 2048, 0),
                                         (70, 96, 256, 5), (513, 300, 192, 40), (64, 777, 1024, 10)])
@pytest.mark.parametrize("wide", [None, 0])
def test_prefill_small(M, N, K, n_out, wide, tune):
    import torch
    if wide is not None:
        tune(qw.QW_TUNE_PREFILL_WIDE_TILES, wide)
    W = inputs.weight(N, K, workload=116)
    perm = np.random.default_rng(M + N).permutation(K).astype(np.int32)
    r = oracle.quantize_int4(W, perm, n_out)
    pw = _pack(W, perm, n_out)
    X = oracle.permute_cols(inputs.act_bf16_bits(M, K, workload=116), perm)
    Y32 = _prefill(pw, X)
    ref = oracle.gemm_prefill_ref(X, oracle.prefill_weight_bf16_int4(r["q"], r["s"], r["W_O"]))
    e = norm_err(Y32.cpu().numpy(), ref)
    print(f"int4 prefill {M}x{N}x{K} anchors={n_out}: err {e:.3e}")
    assert e <= TOL
    Yb = _prefill(pw, X, f32=False)
    np.testing.assert_array_equal(Yb.view(torch.int16).cpu().numpy(),
                                  Y32.to(torch.bfloat16).view(torch.int16).cpu().numpy())


def test_prefill_70b_shape_sampled():
    """2048x8192 times 28672x8192 INT4 (no anchors), sampled outputs; the
    activations are gathered to permuted order on the device."""
    import torch
    M, N, K = 2048, 28672, 8192
    W = inputs.weight(N, K, workload=5)
    perm = np.random.default_rng(5).permutation(K).astype(np.int32)
    pw = _pack(W, perm, 0)
    X = inputs.act_bf16_bits(M, K, workload=5)
    Xp_dev = qw.qw_permute_cols(bf16_dev(X), to_dev(perm))
    Y = qw.qgemm_prefill(pw, Xp_dev, out_dtype=torch.float32).cpu().numpy()
    g = np.random.default_rng(55)
    ms = np.sort(g.choice(M, 48, replace=False))
    ns = np.sort(g.choice(N, 320, replace=False))
    r = oracle.quantize_int4(W[ns], perm, 0)
    ref = oracle.gemm_prefill_ref(oracle.permute_cols(X[ms], perm),
                                  oracle.prefill_weight_bf16_int4(r["q"], r["s"], r["W_O"]))
    e = norm_err(Y[np.ix_(ms, ns)], ref)
    print(f"int4 70B-shaped prefill: sampled err {e:.3e}")
    assert e <= TOL
