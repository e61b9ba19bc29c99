"""GPU parity of the fused decode stack (qw_stack_prepare / qw_stack_run)
with the fp64 oracle. Every stage runs the matrix-core GEMV body in one
persistent launch, with a device-wide barrier between stages. Chained stages
(o reads y_q, down reads y_gate as the run wrote them) check cross-stage
visibility: their reference takes its input from the oracle's own chain
(y_q, y_gate computed by the oracle and rounded to fp16), never from the
device; anchors are the oracle's choice (the device's is checked equal). A
stage with the gated activation (a merged gate/up matrix) feeds the down
projection as a decoder block does. A second run gives the same bits. No
barrier wait may give up."""

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
    idx = oracle.select_outliers(W, X, frac) if frac else None
    if idx is not None:
        dev = qw.qw_select_outliers(Wd, to_dev(X), frac).cpu().numpy()
        np.testing.assert_array_equal(np.sort(dev), np.sort(idx))
    pw = qw.qw_pack(Wd, qw.QW_FMT_2BIT_G32, None if idx is None else to_dev(np.asarray(idx, np.int32)))
    torch.cuda.synchronize()
    return W, pw, idx


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


def _oracle_y(pw_w_idx, x16):
    W, pw, idx = pw_w_idx
    r = oracle.quantize_2bit(W, idx)
    return oracle.gemv_2bit_ref(np.asarray(x16, np.float16)[None, :], r["q"], r["S"], r["Z"], r["idx"], r["W_O"])[0]


@pytest.mark.parametrize("L", [1, 3])
def test_stack_chained_layers_match_oracle(L):
    import torch
    layers, stages = _stages(L, torch.float16)
    st = qw.Stack(stages)
    st.run()
    torch.cuda.synchronize()
    assert st.error() == 0
    for li, (w, x_attn, x_mlp, x_down, y) in enumerate(layers):
        xa = x_attn.cpu().numpy()
        xm = x_mlp.cpu().numpy()
        ref = {n: _oracle_y(w[n], xa) for n in ("q", "k", "v")}
        ref.update({n: _oracle_y(w[n], xm) for n in ("gate", "up")})
        # the chained inputs as the oracle computes them, rounded to fp16
        ref["o"] = _oracle_y(w["o"], oracle.fp16_rne(ref["q"]))
        ref["down"] = _oracle_y(w["down"], oracle.fp16_rne(ref["gate"]))
        for n in ("q", "k", "v", "o", "gate", "up", "down"):
            e = norm_err(y[n].float().cpu().numpy()[None, :], ref[n][None, :])
            print(f"layer {li} {n}: err {e:.3e}")
            assert e <= TOL, (li, n, e)
    # a second run gives the same bits (sync cleared by each run)
    first = [[t.clone() for t in ys] for _, _, ys in stages]
    st.run()
    torch.cuda.synchronize()
    assert st.error() == 0
    for (_, _, ys), f in zip(stages, first):
        for t, ft in zip(ys, f):
            assert torch.equal(t, ft)


@pytest.mark.parametrize("L", [1, 2])
def test_stack_swiglu_feeds_down(L):
    """Per layer: q/k/v, o (reads y_q), the merged gate/up stage writing
    silu(gate) * up (fp16), and down reading it: the MLP half of a decoder
    block as it runs per token."""
    import torch
    stages, layers = [], []
    for l in range(L):
        s = 300 + 10 * l
        w = {n: _packed(N, K, s + i) for i, (n, N, K) in enumerate(
            [("q", H, H), ("k", KV, H), ("v", KV, H), ("o", H, H), ("gateup", 2 * I, H), ("down", H, I)])}
        x_attn = f16_dev(inputs.act_f16(1, H, workload=s)[0])
        x_mlp = f16_dev(inputs.act_f16(1, H, workload=s + 7)[0])
        y = {n: torch.zeros(H if n in ("q", "o", "down") else (KV if n in ("k", "v") else I),
                            dtype=torch.float16, device="cuda") for n in w}
        stages.append(([w["q"][1], w["k"][1], w["v"][1]], x_attn, [y["q"], y["k"], y["v"]]))
        stages.append(([w["o"][1]], y["q"], [y["o"]]))
        stages.append(([w["gateup"][1]], x_mlp, [y["gateup"]], True))
        stages.append(([w["down"][1]], y["gateup"], [y["down"]]))
        layers.append((w, x_attn, x_mlp, y))
    st = qw.Stack(stages)
    st.run()
    torch.cuda.synchronize()
    assert st.error() == 0
    for li, (w, x_attn, x_mlp, y) in enumerate(layers):
        xm = x_mlp.cpu().numpy()
        Wg, _, idx = w["gateup"]
        r = oracle.quantize_2bit(Wg, idx)
        act = oracle.gemv_2bit_swiglu_ref(np.asarray(xm, np.float16)[None, :], r["q"], r["S"], r["Z"],
                                          r["idx"], r["W_O"])[0]
        ref_down = _oracle_y(w["down"], oracle.fp16_rne(act))
        e_act = norm_err(y["gateup"].float().cpu().numpy()[None, :], act[None, :])
        e_down = norm_err(y["down"].float().cpu().numpy()[None, :], ref_down[None, :])
        print(f"layer {li}: silu(gate)*up err {e_act:.3e}, down err {e_down:.3e}")
        assert e_act <= TOL and e_down <= TOL
    first = [[t.clone() for t in ys] for _, _, ys, *_ in stages]
    st.run()
    torch.cuda.synchronize()
    assert st.error() == 0
    for (_, _, ys, *_), f in zip(stages, first):
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
    with pytest.raises(ValueError):  # one merged weight per swiglu stage
        qw.Stack([([pw, pw], x, [y, y], True)])
    _, pw3, _ = _packed(48, 1024, 252, frac=0)  # N = 48: not two halves of whole tiles
    y3 = torch.zeros(24, dtype=torch.float16, device="cuda")
    with pytest.raises(qw.QwError) as e:
        qw.Stack([([pw3], x, [y3], True)])
    assert e.value.status == qw.QW_ERR_INVALID_ARG
