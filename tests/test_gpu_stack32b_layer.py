"""Decoder layers of the 32B-shaped decode stack at their full size (hidden
5120, intermediate 27648, 40 query / 8 KV heads of 128, 2-bit G32 with 3.5%
anchors), in the two launch configurations the benchmark times: grouped
launches (q/k/v and gate/up grouped) and the fused persistent stack. Two
layers are checked (the first and the last of 64). For every projection the
anchor channels are the oracle's own selection (section 4 of the OTF-LLM
page: top 3.5% by |W| x |X_profile| from that input's seeded profile), and
the device's selection from the same profile must equal it: 179 of 5120
channels for q/k/v/o/gate/up (gate/up over 27648 rows), 967 of 27648 for
down. An output row depends only on its own weight row and the anchor set,
so 256 sampled rows of every projection are checked against the fp64
oracle."""

import numpy as np
import pytest

import oracle
from bit_weight_quantized_qw_amd import inputs, qw
from gpu_util import TOL, norm_err, to_dev, f16_dev

pytestmark = pytest.mark.gpu

H, I, KV = 5120, 27648, 1024
PROJ = [("q", H, H, 0), ("k", KV, H, 0), ("v", KV, H, 0), ("o", H, H, 1),
        ("gate", I, H, 2), ("up", I, H, 2), ("down", H, I, 3)]


@pytest.fixture(scope="module", params=[0, 63])
def layer(request):
    import torch
    l = request.param
    w, prof, xs = {}, {}, {}
    refs = {}
    for p, (n, N, K, inp) in enumerate(PROJ):
        if inp not in prof:
            prof[inp] = inputs.profile(256, K, workload=4, layer=l, proj=inp)
            xs[inp] = inputs.act_f16(1, K, workload=4, layer=l, proj=inp)
        print(f"layer {l} {n} {N}x{K}: drawing, selecting and packing", flush=True)
        W = inputs.weight(N, K, workload=4, layer=l, proj=p)
        want = oracle.select_outliers(W, prof[inp], 0.035)
        assert len(want) == (967 if K == I else 179)
        Wd = to_dev(W)
        got = qw.qw_select_outliers(Wd, to_dev(prof[inp]), 0.035).cpu().numpy()
        np.testing.assert_array_equal(got, want, err_msg=f"layer {l} anchors of {n} ({N}x{K})")
        pw = qw.qw_pack(Wd, qw.QW_FMT_2BIT_G32, to_dev(want))
        del Wd
        w[n] = (N, pw, inp)
        rows = np.sort(inputs.rng(4, l, 0, 5).choice(N, 256, replace=False))
        r = oracle.quantize_2bit(W[rows], want)
        refs[n] = (rows, oracle.gemv_2bit_ref(xs[inp], r["q"], r["S"], r["Z"], r["idx"], r["W_O"]))
        del W
    torch.cuda.synchronize()
    return w, xs, refs


def test_layer_grouped_launches(layer):
    import torch
    w, xs, refs = layer
    xd = {k: f16_dev(v) for k, v in xs.items()}
    y = {}
    y["q"], y["k"], y["v"] = qw.qgemv_2bit_grouped([w["q"][1], w["k"][1], w["v"][1]], xd[0],
                                                   out_dtype=torch.float32)
    y["o"] = qw.qgemv_2bit(w["o"][1], xd[1], out_dtype=torch.float32)
    y["gate"], y["up"] = qw.qgemv_2bit_grouped([w["gate"][1], w["up"][1]], xd[2], out_dtype=torch.float32)
    y["down"] = qw.qgemv_2bit(w["down"][1], xd[3], out_dtype=torch.float32)
    for n, (rows, r) in refs.items():
        e = norm_err(y[n].cpu().numpy()[:, rows], r)
        print(f"{n} {w[n][1].N}x{w[n][1].K}: err {e:.3e} on {len(rows)} sampled rows")
        assert e <= TOL, (n, e)


def test_layer_fused_stack(layer):
    import torch
    w, xs, refs = layer
    xd = {k: f16_dev(v)[0] for k, v in xs.items()}
    y = {n: torch.zeros(w[n][1].N, dtype=torch.float32, device="cuda") for n in w}
    st = qw.Stack([([w["q"][1], w["k"][1], w["v"][1]], xd[0], [y["q"], y["k"], y["v"]]),
                   ([w["o"][1]], xd[1], [y["o"]]),
                   ([w["gate"][1], w["up"][1]], xd[2], [y["gate"], y["up"]]),
                   ([w["down"][1]], xd[3], [y["down"]])])
    st.run()
    torch.cuda.synchronize()
    assert st.error() == 0
    for n, (rows, r) in refs.items():
        e = norm_err(y[n].cpu().numpy()[None, rows], r)
        print(f"fused {n}: err {e:.3e}")
        assert e <= TOL, (n, e)
