"""HIP graph capture of the library's calls (torch.cuda.CUDAGraph on ROCm):
every entry point's launches go to the caller's stream and allocate nothing,
so a decode or prefill step can be captured once and replayed. Each replay,
with new inputs written and eager work done between replays, must give the
bits of the same calls run eagerly."""

import numpy as np
import pytest

import oracle
from bit_weight_quantized_qw_amd import inputs, qw
from gpu_util import TOL, norm_err, to_dev, f16_dev, bf16_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("valu", ["0", "1"])
def test_graph_replays_equal_eager(valu, tune):
    import torch
    tune(qw.QW_TUNE_GEMV2_PATH, int(valu))  # the GEMV path captured
    K, B, M = 1024, 2, 300
    W0 = inputs.weight(512, K, workload=90, proj=0)
    W1 = inputs.weight(256, K, workload=90, proj=1)
    W2 = inputs.weight(384, K, workload=90, proj=2)
    idx = np.sort(np.random.default_rng(90).choice(K, 35, replace=False)).astype(np.int32)
    pw0 = qw.qw_pack(to_dev(W0), qw.QW_FMT_2BIT_G32, to_dev(idx))
    pw1 = qw.qw_pack(to_dev(W1), qw.QW_FMT_2BIT_G32, None)
    pwn = qw.qw_pack(to_dev(W2), qw.QW_FMT_NF4_B64)
    pwp = qw.qw_pack(to_dev(W1), qw.QW_FMT_2BIT_G32, None)
    x = f16_dev(inputs.act_f16(B, K, workload=90))
    X = bf16_dev(inputs.act_bf16_bits(M, K, workload=90))
    y0 = torch.empty((B, 512), dtype=torch.float32, device="cuda")
    g0 = torch.empty((B, 512), dtype=torch.float32, device="cuda")
    g1 = torch.empty((B, 256), dtype=torch.float32, device="cuda")
    yn = torch.empty((B, 384), dtype=torch.float32, device="cuda")
    yp = torch.empty((M, 256), dtype=torch.float32, device="cuda")
    outs = [y0, g0, g1, yn, yp]

    def seq():
        qw.qgemv_2bit(pw0, x, out=y0)
        qw.qgemv_2bit_grouped([pw0, pw1], x, outs=[g0, g1])
        qw.qgemv_nf4(pwn, x, out=yn)
        qw.qgemm_prefill(pwp, X, out=yp)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    torch.cuda.synchronize()
    for r in range(3):
        xr = inputs.act_f16(B, K, workload=91 + r)
        Xr = inputs.act_bf16_bits(M, K, workload=91 + r)
        x.copy_(f16_dev(xr))
        X.copy_(bf16_dev(Xr))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        seq()  # eager, same inputs
        torch.cuda.synchronize()
        for a, b in zip(got, outs):
            np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
        # and the eager results are right (2-bit with anchors against the oracle)
        r0 = oracle.quantize_2bit(W0, idx)
        ref = oracle.gemv_2bit_ref(xr, r0["q"], r0["S"], r0["Z"], r0["idx"], r0["W_O"])
        assert norm_err(got[0].cpu().numpy(), ref) <= TOL
