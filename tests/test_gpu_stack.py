"""GPU parity of the fused decode stack (qw_stack_prepare / qw_stack_run).
A stage of one matrix is planned exactly as its own launch, so its output
must equal, bit for bit, the matrix-core GEMV launched alone on the same
input, including inputs that an earlier stage of the same run wrote
(device-wide visibility across the barrier). Grouped stages share the
persistent grid in proportion to their tiles (another K split), so they are
checked against the fp64 oracle. No barrier wait may give up."""

import numpy as np
import pytest

import oracle
from bit_weight_quantized_qw_amd import inputs, qw
from gpu_util import TOL, norm_err, to_dev, f16_dev

pytestmark = pytest.mark.gpu

H, I, KV = 1024, 2560, 256


def _packed(N, K, seed, frac=0.035):
    import torch
    W = inputs.weight(N, K, workload=seed)
    X = inputs.profile(32, K, workload=seed)
    Wd = to_dev(W)
    idx = qw.qw_select_outliers(Wd, to_dev(X), frac) if frac else None
    pw = qw.qw_pack(Wd, qw.QW_FMT_2BIT_G32, idx)
    torch.cuda.synchronize()
    return W, pw, (None if idx is None else idx.cpu().numpy())


def _layer(l, y_dtype):
    """Weights, inputs and outputs of one layer: q/k/v share x_attn, o reads
    y_q (chained), gate/up share x_mlp, down reads y_gate (chained)."""
    import torch
    s = 200 + 10 * l
    w = {n: _packed(N, K, s + i) for i, (n, N, K) in enumerate(
        [("q", H, H), ("k", KV, H), ("v", KV, H), ("o", H, H), ("gate", I, H), ("up", I, H), ("down", H, I)])}
    x_attn = f16_dev(inputs.act_f16(1, H, workload=s)[0])
    x_mlp = f16_dev(inputs.act_f16(1, H, workload=s + 7)[0])
    x_down = f16_dev(inputs.act_f16(1, I, workload=s + 8)[0])
    y = {n: torch.zeros(w[n][1].N, dtype=y_dtype, device="cuda") for n in w}
    return w, x_attn, x_mlp, x_down, y


def _stages(L, y_dtype):
    import torch
    layers = [_layer(l, y_dtype) for l in range(L)]
    stages = []
    for w, x_attn, x_mlp, x_down, y in layers:
        # chained inputs need fp16; with fp32 outputs o and down read their
        # own inputs (of their K: H and I)
        yq = y["q"] if y_dtype == torch.float16 else x_attn
        yg = y["gate"] if y_dtype == torch.float16 else x_down
        stages.append(([w["q"][1], w["k"][1], w["v"][1]], x_attn, [y["q"], y["k"], y["v"]]))
        stages.append(([w["o"][1]], yq, [y["o"]]))
        stages.append(([w["gate"][1], w["up"][1]], x_mlp, [y["gate"], y["up"]]))
        stages.append(([w["down"][1]], yg, [y["down"]]))
    return layers, stages


def _oracle_err(pw_w_idx, x16, y):
    W, pw, idx = pw_w_idx
    r = oracle.quantize_2bit(W, idx)
    ref = oracle.gemv_2bit_ref(x16[None, :], r["q"], r["S"], r["Z"], r["idx"], r["W_O"])
    return norm_err(y.float().cpu().numpy()[None, :], ref)


@pytest.mark.parametrize("L", [1, 3])
def test_stack_single_stages_bit_exact_grouped_within_tolerance(L, tune):
    import torch
    layers, stages = _stages(L, torch.float16)
    st = qw.Stack(stages)
    st.run()
    torch.cuda.synchronize()
    assert st.error() == 0
    tune(qw.QW_TUNE_GEMV2_PATH, 0)   # the matrix-core kernel, as in the stack
    for li, (w, x_attn, x_mlp, x_down, y) in enumerate(layers):
        # o reads y_q and down reads y_gate as the fused run left them
        for n, xin in (("o", y["q"]), ("down", y["gate"])):
            ref = qw.qgemv_2bit(w[n][1], xin.view(1, -1))
            np.testing.assert_array_equal(y[n].view(torch.int16).cpu().numpy(),
                                          ref.view(torch.int16).cpu().numpy()[0], err_msg=f"layer {li} {n}")
        xa = x_attn.cpu().numpy()
        xm = x_mlp.cpu().numpy()
        for n, xin in (("q", xa), ("k", xa), ("v", xa), ("gate", xm), ("up", xm)):
            e = _oracle_err(w[n], xin, y[n])
            assert e <= TOL, (li, n, e)
    # a second run gives the same bits (sync cleared by each run)
    first = [[t.clone() for t in ys] for _, _, ys in stages]
    st.run()
    torch.cuda.synchronize()
    assert st.error() == 0
    for (_, _, ys), f in zip(stages, first):
        for t, ft in zip(ys, f):
            assert torch.equal(t, ft)


def test_stack_fp32_outputs_match_oracle():
    """fp32 outputs of an unchained layer against the fp64 oracle."""
    import torch
    layers, stages = _stages(1, torch.float32)
    st = qw.Stack(stages)
    st.run()
    torch.cuda.synchronize()
    assert st.error() == 0
    w, x_attn, x_mlp, x_down, y = layers[0]
    xa = x_attn.cpu().numpy()[None, :]
    xm = x_mlp.cpu().numpy()[None, :]
    xd = x_down.cpu().numpy()[None, :]
    for n, xin in (("q", xa), ("k", xa), ("v", xa), ("o", xa), ("gate", xm), ("up", xm), ("down", xd)):
        W, pw, idx = w[n]
        r = oracle.quantize_2bit(W, idx)
        ref = oracle.gemv_2bit_ref(xin, r["q"], r["S"], r["Z"], r["idx"], r["W_O"])
        e = norm_err(y[n].cpu().numpy()[None, :], ref)
        assert e <= TOL, (n, e)


def test_stack_rejects_bad_stages():
    import torch
    W, pw, _ = _packed(64, 1024, 250, frac=0)
    x = torch.zeros(1024, dtype=torch.float16, device="cuda")
    y = torch.zeros(64, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        qw.Stack([([pw], x, [])])
    W2, pw2, _ = _packed(64, 96, 251, frac=0)   # K % 512 != 0
    x2 = torch.zeros(96, dtype=torch.float16, device="cuda")
    with pytest.raises(qw.QwError) as e:
        qw.Stack([([pw2], x2, [y])])
    assert e.value.status == qw.QW_ERR_UNSUPPORTED
