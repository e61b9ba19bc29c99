"""Shared helpers for the GPU parity tests (not a test module)."""

import numpy as np

import oracle

# Normwise relative error bound for the products (fp32 accumulation, fp16 or
# fp32 output): max |y - ref| / max |ref| <= 1e-3.
TOL = 1e-3
# Regression bound for fp32-output decode GEMVs: the fp32 accumulation alone
# leaves about 1e-5 normwise (measured up to 6e-6 on the 2-bit kernels and
# 1e-7 on NF4/INT4), so a change that loses precision shows here long
# before it reaches TOL.
TOL_F32_GEMV = 5e-5


def norm_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(y)))
    return float(np.max(np.abs(y - ref)) / den)


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def f16_dev(x16):
    import torch
    return to_dev(np.asarray(x16, np.float16).view(np.int16)).view(torch.float16)


def bf16_dev(bits):
    import torch
    return to_dev(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def oracle_2bit(W, idx=None):
    """Oracle quantization in the library's stored layout."""
    r = oracle.quantize_2bit(W, idx)
    return {
        "codes": oracle.pack_2bit(r["q"]),
        "sz": oracle.sz_interleaved(r["S"], r["Z"]),
        "W_O": r["W_O"],
        "q": r["q"], "S": r["S"], "Z": r["Z"], "idx": r["idx"],
    }


def oracle_nf4(W):
    q, a = oracle.quantize_nf4(W)
    return {"codes": oracle.pack_nf4(q), "absmax": a, "q": q}


def assert_bits_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    g = got.view(np.uint8) if got.dtype.itemsize == 1 else got.view(f"u{got.dtype.itemsize}")
    w = want.view(np.uint8) if want.dtype.itemsize == 1 else want.view(f"u{want.dtype.itemsize}")
    bad = np.argwhere(g != w)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}"
