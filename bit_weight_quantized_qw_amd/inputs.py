"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle
checks. This module holds no arithmetic of the method: it only draws random
numbers and rounds them to the input storage types.

Keys: every draw uses ``numpy.random.default_rng([workload, layer, proj,
role])`` with role 0 = weight, 1 = activation, 2 = calibration profile,
3 = spiked channels of the profile. Large weights for the benchmark can be
drawn on the GPU instead (``torch_weight``), from a torch generator seeded
with the same four numbers folded into one integer.
"""

import numpy as np

ROLE_W, ROLE_X, ROLE_PROFILE, ROLE_SPIKE = 0, 1, 2, 3
W_STD = np.float32(0.02)


def rng(workload, layer=0, proj=0, role=0):
    return np.random.default_rng([int(workload), int(layer), int(proj), int(role)])


def weight(N, K, workload, layer=0, proj=0):
    """fp32 (N, K) with entries N(0, 0.02^2)."""
    g = rng(workload, layer, proj, ROLE_W)
    return g.standard_normal((N, K), dtype=np.float32) * W_STD


def act_f16(B, K, workload, layer=0, proj=0):
    """fp16 (B, K) activations N(0, 1), rounded from fp32."""
    g = rng(workload, layer, proj, ROLE_X)
    return g.standard_normal((B, K), dtype=np.float32).astype(np.float16)


def act_bf16_bits(M, K, workload, layer=0, proj=0):
    """bf16 bit patterns (uint16, (M, K)) of N(0, 1) activations, rounded to
    nearest-even from fp32 by torch."""
    import torch
    g = rng(workload, layer, proj, ROLE_X)
    x32 = torch.from_numpy(g.standard_normal((M, K), dtype=np.float32))
    return x32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def profile(P, K, workload, layer=0, proj=0, spike_frac=0.01, spike_gain=20.0):
    """fp32 (P, K) calibration activations N(0, 1) in which floor(spike_frac*K)
    channels, chosen without replacement, are scaled by ``spike_gain``."""
    g = rng(workload, layer, proj, ROLE_PROFILE)
    X = g.standard_normal((P, K), dtype=np.float32)
    n = int(np.floor(spike_frac * K))
    if n:
        ch = rng(workload, layer, proj, ROLE_SPIKE).choice(K, n, replace=False)
        X[:, ch] *= np.float32(spike_gain)
    return X


def special_weight(kind, N, K, workload=0):
    """Structured fp32 weights for edge cases: 'const' (one value per group
    of 32), 'zero', 'alternating' (+a/-a), 'ramp' (monotone along K)."""
    g = rng(workload, 0, 0, ROLE_W)
    if kind == "zero":
        return np.zeros((N, K), np.float32)
    if kind == "const":
        v = g.standard_normal((N, K // 32, 1), dtype=np.float32) * W_STD
        return np.repeat(v, 32, axis=2).reshape(N, K)
    if kind == "alternating":
        a = np.abs(g.standard_normal((N, 1), dtype=np.float32)) * W_STD + np.float32(1e-3)
        s = np.where(np.arange(K) % 2 == 0, 1.0, -1.0).astype(np.float32)
        return a * s[None, :]
    if kind == "ramp":
        return (np.arange(K, dtype=np.float32)[None, :] * np.float32(1e-4)
                + g.standard_normal((N, 1), dtype=np.float32) * W_STD)
    raise ValueError(kind)


def torch_seed(workload, layer=0, proj=0, role=0):
    return ((int(workload) * 1009 + int(layer)) * 1013 + int(proj)) * 7 + int(role)


def torch_weight(N, K, workload, layer=0, proj=0, device="cuda"):
    """fp32 (N, K) N(0, 0.02^2) drawn on ``device`` by torch (for sizes where a
    host draw is too slow). Not the same numbers as ``weight``."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(workload, layer, proj, ROLE_W))
    w = torch.randn((N, K), generator=gen, device=device, dtype=torch.float32)
    return w.mul_(float(W_STD))


def torch_profile(P, K, workload, layer=0, proj=0, spike_frac=0.01,
                  spike_gain=20.0, device="cuda"):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(workload, layer, proj, ROLE_PROFILE))
    X = torch.randn((P, K), generator=gen, device=device, dtype=torch.float32)
    n = int(np.floor(spike_frac * K))
    if n:
        ch = rng(workload, layer, proj, ROLE_SPIKE).choice(K, n, replace=False)
        X[:, torch.as_tensor(ch, device=device)] *= spike_gain
    return X
