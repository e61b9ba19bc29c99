"""qgemv_2bit_static: the 2-bit GEMV variant that allocates nothing, its K-split
partial rows in the library's static device array instead of a caller
workspace. Called through the C ABI and compared bit for bit with
qgemv_2bit_ws (the entry point it varies) on the same inputs: two calls in a
row that both run as K parts, the second smaller (so it reads only what it
wrote over the first call's leftovers), a call that needs no scratch, and a
request beyond the array's size, refused before any launch."""

import ctypes

import numpy as np
import pytest

from bit_weight_quantized_qw_amd import inputs, qw
from gpu_util import to_dev, f16_dev

pytestmark = pytest.mark.gpu


def _packed(N, K, n_anchor, seed):
    W = inputs.weight(N, K, workload=seed)
    idx = np.sort(np.random.default_rng(seed).choice(K, n_anchor, replace=False)).astype(np.int32)
    return qw.qw_pack(to_dev(W), qw.QW_FMT_2BIT_G32, to_dev(idx))


def _static_call(pw, x, y):
    """Direct C-ABI call of qgemv_2bit_static; returns the status."""
    import torch
    v = pw.view()
    return qw.lib().qgemv_2bit_static(ctypes.byref(v), ctypes.c_void_p(x.data_ptr()), x.shape[0],
                                      ctypes.c_void_p(y.data_ptr()), qw.QW_DT_F32,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_static_scratch_equals_workspace_twice_then_smaller():
    import torch
    K = 27648
    cases = [(1536, 900, 8, 97), (520, 300, 3, 98)]  # second: fewer rows, fewer batch rows
    for N, n_anchor, B, seed in cases:
        pw = _packed(N, K, n_anchor, seed)
        need = qw.qgemv_2bit_workspace_bytes(pw, B)
        assert 0 < need <= qw.QW_STATIC_SCRATCH_BYTES, need
        x = f16_dev(inputs.act_f16(B, K, workload=seed))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        want = qw.qgemv_2bit_ws(pw, x, ws, out_dtype=torch.float32)
        y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
        assert _static_call(pw, x, y) == qw.QW_OK
        torch.cuda.synchronize()
        assert torch.equal(y, want), (N, B)


def test_static_without_scratch_need_equals_plain_call():
    import torch
    N, K, B = 700, 5120, 2
    pw = _packed(N, K, 179, 99)
    assert qw.qgemv_2bit_workspace_bytes(pw, B) == 0
    x = f16_dev(inputs.act_f16(B, K, workload=99))
    want = qw.qgemv_2bit(pw, x, out_dtype=torch.float32)
    y = torch.empty((B, N), dtype=torch.float32, device="cuda")
    assert _static_call(pw, x, y) == qw.QW_OK
    torch.cuda.synchronize()
    assert torch.equal(y, want)


def test_static_refuses_beyond_its_array():
    """A shape whose K parts need more than the static array: refused with
    QW_ERR_SCRATCH_LIMIT before any launch (y keeps its fill)."""
    import torch
    N, K, B = 65536, 27648, 8
    z = qw.qw_packed_sizes(qw.QW_FMT_2BIT_G32, N, K, 0)
    pw = qw.PackedWeight(qw.QW_FMT_2BIT_G32, N, K, 0)
    pw.codes.zero_()
    pw.scales.zero_()
    assert pw.codes.numel() == z["codes"]
    need = qw.qgemv_2bit_workspace_bytes(pw, B)
    assert need > qw.QW_STATIC_SCRATCH_BYTES, need
    x = torch.zeros((B, K), dtype=torch.float16, device="cuda")
    y = torch.full((B, N), 7.0, dtype=torch.float32, device="cuda")
    assert _static_call(pw, x, y) == qw.QW_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
