"""GPU parity of the K-split matrix-core 2-bit GEMV (qgemv_2bit_ws with a
caller-owned workspace). A matrix's channels are cut into equal parts of
whole 512-channel super-chunks and its anchor chunks into runs, one part per
matrix of a grouped launch (two launches beyond four parts); the parts' fp32
partial rows are written to the workspace and added in order. Part counts
forced through the QW_TUNE_GEMV2_SPLIT hook on small ragged shapes (parts
with and without anchors, batches 1-8), a one-hot check that every part
reads its own channels, and the automatic choice at 5120x27648 with 967
anchors (where batches of 2-8 only fit as parts), all against the fp64
oracle; the anchor channels chosen on the device equal the oracle's own
selection there and at 8192x28672 (1003 anchors). Without a workspace the
same calls run one row group at a time and stay within the bound."""

import numpy as np
import pytest

import oracle
from bit_weight_quantized_qw_amd import inputs, qw
from gpu_util import TOL, norm_err, to_dev, f16_dev

pytestmark = pytest.mark.gpu


def _packed(W, idx):
    idd = to_dev(np.asarray(idx, np.int32)) if idx is not None and len(idx) else None
    return qw.qw_pack(to_dev(W), qw.QW_FMT_2BIT_G32, idd)


def _run(pw, x16, f32, workspace=True):
    """qgemv_2bit_ws with a workspace of the size the library asks for (or
    none: then the call runs as qgemv_2bit)."""
    import torch
    xd = f16_dev(x16)
    ws = qw.gemv_workspace(pw, xd.shape[0]) if workspace else None
    y = qw.qgemv_2bit_ws(pw, xd, ws, out_dtype=torch.float32 if f32 else torch.float16)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def _anchors(K, n, seed):
    if n == 0:
        return None
    return np.sort(np.random.default_rng(seed).choice(K, n, replace=False)).astype(np.int32)


@pytest.mark.parametrize("N,K,n_anchor,ks", [
    (200, 3072, 107, 2), (200, 3072, 107, 3), (200, 3072, 107, 6),
    (77, 3072, 614, 3), (77, 3072, 614, 6),
    (48, 4608, 0, 3), (33, 6144, 2000, 4), (33, 6144, 2000, 6)])
@pytest.mark.parametrize("B", [1, 3, 8])
def test_forced_split_matches_oracle(N, K, n_anchor, ks, B, tune):
    tune(qw.QW_TUNE_GEMV2_PATH, 0)
    tune(qw.QW_TUNE_GEMV2_SPLIT, ks)
    W = inputs.weight(N, K, workload=90)
    idx = _anchors(K, n_anchor, N + K)
    x = inputs.act_f16(B, K, workload=90)
    pw = _packed(W, idx)
    r = oracle.quantize_2bit(W, idx)
    ref = oracle.gemv_2bit_ref(x, r["q"], r["S"], r["Z"], r["idx"], r["W_O"])
    y32 = _run(pw, x, True)
    y16 = _run(pw, x, False)
    e = norm_err(y32, ref)
    print(f"{N}x{K} anchors={n_anchor} parts={ks} B={B}: err {e:.3e}")
    assert e <= TOL
    # the fp16 output is the fp32 sum of the parts rounded once
    np.testing.assert_array_equal(y16.astype(np.float16), y32.astype(np.float16))


def test_split_parts_read_their_own_channels(tune):
    tune(qw.QW_TUNE_GEMV2_PATH, 0)
    tune(qw.QW_TUNE_GEMV2_SPLIT, 3)
    N, K = 40, 3072
    W = inputs.weight(N, K, workload=91)
    idx = np.array([5, 700, 1500, 2047, 3000] + list(range(2100, 2400, 3)), np.int32)
    idx = np.unique(idx)
    pw = _packed(W, idx)
    r = oracle.quantize_2bit(W, idx)
    Wh = oracle.dequant_2bit(r["q"], r["S"], r["Z"])
    cols = [0, 5, 511, 512, 1023, 1024, 1500, 2047, 2048, 2100, 2103, 2397, 3000, 3071]
    x = np.zeros((len(cols), K), np.float16)
    for b, k in enumerate(cols[:8]):
        x[b, k] = 1
    x2 = np.zeros((len(cols) - 8, K), np.float16)
    for b, k in enumerate(cols[8:]):
        x2[b, k] = 1
    y = np.concatenate([_run(pw, x[:8], True), _run(pw, x2, True)])
    pos = {int(c): i for i, c in enumerate(idx)}
    for b, k in enumerate(cols):
        ref = r["W_O"][:, pos[k]].astype(np.float64) if k in pos else Wh[:, k]
        assert norm_err(y[b], ref) <= 1e-6, k


def test_split_fp16_inputs_at_extremes(tune):
    """Large and tiny inputs through the parts (per-group scaling of x)."""
    tune(qw.QW_TUNE_GEMV2_PATH, 0)
    tune(qw.QW_TUNE_GEMV2_SPLIT, 2)
    N, K = 64, 2048
    W = inputs.weight(N, K, workload=92)
    idx = _anchors(K, 70, 92)
    pw = _packed(W, idx)
    r = oracle.quantize_2bit(W, idx)
    for scale in (1e-4, 3000.0):
        x = np.clip(inputs.act_f16(2, K, workload=92).astype(np.float32) * scale, -65504, 65504)
        x = x.astype(np.float16)
        ref = oracle.gemv_2bit_ref(x, r["q"], r["S"], r["Z"], r["idx"], r["W_O"])
        e = norm_err(_run(pw, x, True), ref)
        assert e <= TOL, (scale, e)


@pytest.fixture(scope="module")
def down():
    """The 32B down projection (5120x27648, 967 anchors): the anchors are the
    oracle's own selection (section 4 of the OTF-LLM page), and the device's
    selection from the same profile must equal it."""
    N, K = 5120, 27648
    W = inputs.weight(N, K, workload=4, layer=0, proj=6)
    X = inputs.profile(256, K, workload=4, layer=0, proj=3)
    want = oracle.select_outliers(W, X, 0.035)
    assert len(want) == 967
    Wd = to_dev(W)
    got = qw.qw_select_outliers(Wd, to_dev(X), 0.035).cpu().numpy()
    np.testing.assert_array_equal(got, want, err_msg="device anchor set at 5120x27648")
    pw = qw.qw_pack(Wd, qw.QW_FMT_2BIT_G32, to_dev(want))
    del Wd
    rows = np.sort(inputs.rng(4, 0, 6, 5).choice(N, 192, replace=False))
    r = oracle.quantize_2bit(W[rows], want)
    return pw, rows, r


def test_selection_down70b_equals_oracle():
    """8192x28672 with a 28672-channel profile: 1003 anchors, the device's
    choice equals the oracle's."""
    N, K = 8192, 28672
    W = inputs.weight(N, K, workload=6)
    X = inputs.profile(256, K, workload=6)
    want = oracle.select_outliers(W, X, 0.035)
    assert len(want) == 1003
    got = qw.qw_select_outliers(to_dev(W), to_dev(X), 0.035).cpu().numpy()
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("B", [1, 2, 5, 8])
@pytest.mark.parametrize("path", ["auto", "matrix_core"])
def test_down_projection_batches(down, B, path, tune):
    """5120x27648 with 967 anchors: batches of 2-8 run as K parts (their x
    does not fit one workgroup whole); checked on 192 sampled rows. Without
    a workspace (qgemv_2bit) the same call runs without parts."""
    if path == "matrix_core":
        tune(qw.QW_TUNE_GEMV2_PATH, 0)
    pw, rows, r = down
    x = inputs.act_f16(B, 27648, workload=4, layer=0, proj=9)
    ref = oracle.gemv_2bit_ref(x, r["q"], r["S"], r["Z"], r["idx"], r["W_O"])
    for ws in (True, False):
        y = _run(pw, x, True, workspace=ws)
        e = norm_err(y[:, rows], ref)
        print(f"down B={B} {path} workspace={ws}: err {e:.3e}")
        assert e <= TOL


def test_workspace_query_and_small_workspace():
    """The library asks for a workspace exactly where the batch needs K parts
    (parts * B * N * 4 bytes), and a workspace one byte short runs the call
    as qgemv_2bit does, bit for bit."""
    import torch
    N, K = 64, 27648
    W = inputs.weight(N, K, workload=96)
    pw = _packed(W, _anchors(K, 500, 96))
    assert qw.qgemv_2bit_workspace_bytes(pw, 1) == 0
    for B in (2, 8):
        nb = qw.qgemv_2bit_workspace_bytes(pw, B)
        assert nb > 0 and nb % (B * N * 4) == 0 and nb // (B * N * 4) <= 8, (B, nb)
        x = f16_dev(inputs.act_f16(B, K, workload=96))
        plain = qw.qgemv_2bit(pw, x, out_dtype=torch.float32)
        short = torch.empty(nb - 1, dtype=torch.uint8, device="cuda")
        got = qw.qgemv_2bit_ws(pw, x, short, out_dtype=torch.float32)
        assert torch.equal(got, plain), B


def test_split_call_in_graph_replays_equal_eager(down):
    """A K-split call captured in a HIP graph replays with the eager call's
    bits, for new inputs copied in between replays and with other work
    between them (the workspace is allocated before the capture)."""
    import torch
    pw, _, _ = down
    B = 8
    ws = qw.gemv_workspace(pw, B)
    assert ws is not None
    xs = [f16_dev(inputs.act_f16(B, 27648, workload=4, layer=0, proj=20 + i)) for i in range(3)]
    eager = [qw.qgemv_2bit_ws(pw, xi, ws, out_dtype=torch.float32).clone() for xi in xs]
    x = torch.empty_like(xs[0])
    y = torch.zeros((B, 5120), dtype=torch.float32, device="cuda")
    x.copy_(xs[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qw.qgemv_2bit_ws(pw, x, ws, out=y)
    for rep in range(2):
        for i, xi in enumerate(xs):
            x.copy_(xi)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, eager[i]), (rep, i)
            float((xi.float() * 2).sum())


def test_binding_rejects_mismatched_shapes():
    """The library reads B x K of x and writes B x N of y: the binding refuses
    tensors of other shapes before any launch."""
    import torch
    W = inputs.weight(64, 1024, workload=93)
    pw = _packed(W, None)
    x = torch.zeros((2, 1024), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        qw.qgemv_2bit(pw, torch.zeros((2, 512), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        qw.qgemv_2bit(pw, x, out=torch.zeros((1, 64), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        qw.qgemv_2bit_grouped([pw, pw], x, outs=[torch.zeros((2, 64), dtype=torch.float16, device="cuda")])


def test_grouped_call_of_split_matrices_equals_separate_calls():
    """Matrices that run as K parts (batch 2 at K = 27648) in one grouped
    call: each is launched alone, so the outputs equal separate calls."""
    import torch
    K = 27648
    pws = []
    for p, N in enumerate((100, 40)):
        W = inputs.weight(N, K, workload=94, proj=p)
        pws.append(_packed(W, _anchors(K, 300, 94 + p)))
    x = f16_dev(inputs.act_f16(2, K, workload=94))
    ys = qw.qgemv_2bit_grouped(pws, x, out_dtype=torch.float32)
    for pw, yg in zip(pws, ys):
        ysep = qw.qgemv_2bit(pw, x, out_dtype=torch.float32)
        np.testing.assert_array_equal(yg.cpu().numpy(), ysep.cpu().numpy())


@pytest.mark.parametrize("forced", ["5", "9", "1"])
def test_invalid_forced_part_count_falls_back(forced, tune):
    """A forced part count that does not divide the super-chunks or does not
    fit (or 1 where the batch cannot run whole) leaves the automatic choice,
    bit for bit."""
    import torch
    N, K = 64, 27648
    W = inputs.weight(N, K, workload=95)
    pw = _packed(W, _anchors(K, 500, 95))
    x = f16_dev(inputs.act_f16(4, K, workload=95))
    ws = torch.empty(8 * 4 * N * 4, dtype=torch.uint8, device="cuda")  # room for 8 parts
    auto = qw.qgemv_2bit_ws(pw, x, ws, out_dtype=torch.float32).cpu().numpy()
    tune(qw.QW_TUNE_GEMV2_SPLIT, int(forced))
    got = qw.qgemv_2bit_ws(pw, x, ws, out_dtype=torch.float32).cpu().numpy()
    np.testing.assert_array_equal(got, auto)
