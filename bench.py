#!/usr/bin/env python3
"""Throughput of the fused low-bit dequant GEMV / prefill GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

Prints ONE JSON line. A step is one pass of the hot path over one batch of
synthetic input for the chosen workload:

  decode32b_stack (default) -- one token through the 448 projection GEMVs of
      a 64-layer 32B-shaped decoder (q/k/v grouped per launch; gate and up as
      one merged matrix whose launch writes silu(gate) * up, read by down),
      2-bit G32 with 3.5% fp16 anchors, 13.9 GB of weights per token. The
      line also carries a ``prefill`` object: the 70B-shaped 2-bit prefill
      GEMM (2048x8192 bf16 times 28672x8192) timed in the same run, so both
      halves of the metric (GEMV GB/s, prefill TFLOP/s) come from one run;
  llama7b_mlp_up_gemv     -- W 11008x4096 N(0, 0.02^2), batch-1 fp16
      activations; one NF4 (block 64) GEMV and one 2-bit (group 32) GEMV of
      the same matrix;
  single_layer_2048       -- 2-bit GEMV 2048x2048, batch 1, no anchors;
  decode14b_b{1,2,4,8}    -- 2-bit GEMV 13824x5120 with 179 fp16 anchors;
  down70b_b{1,8}          -- 2-bit GEMV 8192x28672 with 1003 fp16 anchors (a
      70B-shaped down projection); batch 8 runs as K parts (qgemv_2bit_ws
      with a caller-owned workspace);
  decode32b_stack_fused   -- the same token as one persistent launch with a
      device-wide barrier between its 256 stages;
  decode14b_int4_b{1,8}   -- the v3.2 INT4 format at 13824x5120: channels
      permuted by descending outlier score, the top 1% (51) as fp16 anchors,
      activations given in permuted order;
  prefill70b_nf4 / prefill70b_2bit / prefill70b_int4 -- 2048x8192 bf16 times
      28672x8192 (INT4: X in permuted channel order);
  prep_llama7b_refine5    -- preparing the 11008x4096 weight from fp16: device
      profile sums over 256 calibration rows, 3.5% anchor selection, 2-bit
      pack with 5 refinement rounds (value: fp16 weight GB/s; the packer is
      bound by fp64 arithmetic, its roofline is the fp64 vector peak);
  copy_calib              -- a plain device copy of 1 GiB (counter scale).

Timing: after W untimed steps, two timed passes over exactly K steps, each
bracketed by HIP events with synchronization on both sides.
  - Kernel pass: the K steps are enqueued eagerly behind a GPU sleep; every
    launch carries a pair of HIP events that the library attaches to its own
    kernel dispatch (qw_time_next_call), so the pair brackets the kernel's
    execution alone. roofline.achieved = the dominant kernel's algorithmic
    amount per launch / its average duration from those pairs (the figure a
    kernel trace reports).
  - Step pass: C consecutive steps (the largest divisor of K within 2048
    launches) are captured in a HIP graph and replayed K / C times, as a
    decode loop would issue them. value = algorithmic bytes (GEMV) or flops
    (GEMM) of K steps / time between the events around the replays.
Each GEMV weight set is rotated over copies totalling >= 1 GiB so HBM, not
the 256 MB last-level cache, serves it (the captured steps carry their own
copies). cpu_baseline times the fp64 oracle on the host (product path from
packed arrays) on a bounded sample.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused 2-bit dequant-GEMV achieved HBM GB/s and % of peak; prefill GEMM TFLOP/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP64_PEAK_TFLOPS = 78.6
ROTATE_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- workloads

class Workload:
    """launches(i): list of (kernel_name, callable) making up step i."""
    name = ""
    steps, warmup = 200, 20  # defaults when the command line gives none
    library = True  # every launch is one libqw entry-point call
    # whole-step time from replays of steps captured in a HIP graph (the
    # per-launch kernel times still come from the eager pass)
    graph = True
    unit = "GB/s"
    bound = "hbm"
    dtype = "f16"

    def launches(self, i):
        raise NotImplementedError

    def step_amount(self):  # bytes or flops per step (algorithmic)
        raise NotImplementedError

    def kernel_amount(self):  # per-launch algorithmic amount by kernel name
        raise NotImplementedError

    def kernel_bytes(self):  # per-launch algorithmic bytes by kernel name
        return self.kernel_amount() if self.unit == "GB/s" else {}

    def config(self):
        raise NotImplementedError

    def cpu_baseline(self):
        return None


def _gemv2_bytes(N, K, n_out, B):
    pad = (n_out + 7) // 8 * 8 if n_out else 0
    return N * K // 4 + N * (K // 32) * 4 + N * pad * 2 + n_out * 4 + B * K * 2 + B * N * 2


def _nf4_bytes(N, K, B):
    return N * K // 2 + N * (K // 64) * 4 + B * K * 2 + B * N * 2


def _int4_bytes(N, K, n_out, B):
    pad = (n_out + 7) // 8 * 8 if n_out else 0
    return N * K // 2 + N * (K // 32) * 2 + N * pad * 2 + B * K * 2 + B * N * 2


def _copies(pw, n):
    """n independent device copies of a packed weight (for cache rotation)."""
    import copy
    out = [pw]
    for _ in range(n - 1):
        c = copy.copy(pw)
        c.codes = pw.codes.clone()
        c.scales = pw.scales.clone()
        if pw.n_out:
            c.out_idx = pw.out_idx.clone()
            c.out_w = pw.out_w.clone()
        out.append(c)
    return out


class Llama7bMlpUp(Workload):
    name = "llama7b_mlp_up_gemv"
    N, K, B = 11008, 4096, 1

    def __init__(self):
        import torch
        from bit_weight_quantized_qw_amd import inputs, qw
        self.qw = qw
        self.Wh = inputs.weight(self.N, self.K, workload=2)
        self.xh = inputs.act_f16(self.B, self.K, workload=2)
        W = torch.from_numpy(self.Wh).cuda()
        p2 = qw.qw_pack(W, qw.QW_FMT_2BIT_G32)
        p4 = qw.qw_pack(W, qw.QW_FMT_NF4_B64)
        del W
        per = p2.nbytes() + p4.nbytes()
        self.R = max(2, math.ceil(ROTATE_BYTES / per))
        self.p2 = _copies(p2, self.R)
        self.p4 = _copies(p4, self.R)
        self.x = torch.from_numpy(self.xh.view(np.int16)).cuda().view(torch.float16)
        self.y2 = torch.empty((self.B, self.N), dtype=torch.float16, device="cuda")
        self.y4 = torch.empty_like(self.y2)

    def launches(self, i):
        r = i % self.R
        return [("qgemv_nf4", lambda: self.qw.qgemv_nf4(self.p4[r], self.x, out=self.y4)),
                ("qgemv_2bit", lambda: self.qw.qgemv_2bit(self.p2[r], self.x, out=self.y2))]

    def kernel_amount(self):
        return {"qgemv_nf4": _nf4_bytes(self.N, self.K, self.B),
                "qgemv_2bit": _gemv2_bytes(self.N, self.K, 0, self.B)}

    def step_amount(self):
        return sum(self.kernel_amount().values())

    def config(self):
        return {"workload": self.name, "N": self.N, "K": self.K, "batch": self.B,
                "formats": ["nf4_b64", "2bit_g32"], "rotate_copies": self.R}

    def cpu_baseline(self):
        import oracle
        r = oracle.quantize_2bit(self.Wh)
        c2, S, Z = oracle.pack_2bit(r["q"]), r["S"], r["Z"]
        q4, a4 = oracle.quantize_nf4(self.Wh)
        c4 = oracle.pack_nf4(q4)

        def one():
            oracle.gemv_nf4_ref(self.xh, oracle.unpack_nf4(c4), a4)
            oracle.gemv_2bit_ref(self.xh, oracle.unpack_2bit(c2), S, Z)
        return _time_oracle(one, self.step_amount(), f"full {self.N}x{self.K} steps (NF4 + 2-bit GEMV, batch 1)")


class SingleLayer2048(Workload):
    name = "single_layer_2048"
    N = K = 2048

    def __init__(self):
        import torch
        from bit_weight_quantized_qw_amd import inputs, qw
        self.qw = qw
        self.Wh = inputs.weight(self.N, self.K, workload=1)
        self.xh = inputs.act_f16(1, self.K, workload=1)
        p = qw.qw_pack(torch.from_numpy(self.Wh).cuda(), qw.QW_FMT_2BIT_G32)
        self.R = max(2, math.ceil(ROTATE_BYTES / p.nbytes()))
        self.p = _copies(p, self.R)
        self.x = torch.from_numpy(self.xh.view(np.int16)).cuda().view(torch.float16)
        self.y = torch.empty((1, self.N), dtype=torch.float16, device="cuda")

    def launches(self, i):
        r = i % self.R
        return [("qgemv_2bit", lambda: self.qw.qgemv_2bit(self.p[r], self.x, out=self.y))]

    def kernel_amount(self):
        return {"qgemv_2bit": _gemv2_bytes(self.N, self.K, 0, 1)}

    def step_amount(self):
        return self.kernel_amount()["qgemv_2bit"]

    def config(self):
        return {"workload": self.name, "N": self.N, "K": self.K, "batch": 1,
                "formats": ["2bit_g32"], "rotate_copies": self.R}

    def cpu_baseline(self):
        import oracle
        r = oracle.quantize_2bit(self.Wh)
        c2 = oracle.pack_2bit(r["q"])
        return _time_oracle(lambda: oracle.gemv_2bit_ref(self.xh, oracle.unpack_2bit(c2), r["S"], r["Z"]),
                            self.step_amount(), "full 2048x2048 steps")


class Decode14b(Workload):
    N, K = 13824, 5120
    SEED, PREFIX = 3, "decode14b"
    ORACLE_ROWS = None  # rows the CPU baseline computes (None: all)

    def __init__(self, B):
        import torch
        from bit_weight_quantized_qw_amd import inputs, qw
        self.qw, self.B = qw, B
        self.name = f"{self.PREFIX}_b{B}"
        self.Wh = inputs.weight(self.N, self.K, workload=self.SEED)
        Xp = inputs.profile(256, self.K, workload=self.SEED)
        self.Xp = Xp
        Wd = torch.from_numpy(self.Wh).cuda()
        idx = qw.qw_select_outliers(Wd, torch.from_numpy(Xp).cuda(), 0.035)
        self.n_out = int(idx.numel())
        p = qw.qw_pack(Wd, qw.QW_FMT_2BIT_G32, idx)
        del Wd
        self.R = max(2, math.ceil(ROTATE_BYTES / p.nbytes()))
        self.p = _copies(p, self.R)
        self.xh = inputs.act_f16(B, self.K, workload=self.SEED)
        self.x = torch.from_numpy(self.xh.view(np.int16)).cuda().view(torch.float16)
        self.y = torch.empty((B, self.N), dtype=torch.float16, device="cuda")
        # caller-owned K-split workspace (None where the batch runs whole)
        self.ws = qw.gemv_workspace(self.p[0], B)

    def launches(self, i):
        r = i % self.R
        return [("qgemv_2bit", lambda: self.qw.qgemv_2bit_ws(self.p[r], self.x, self.ws, out=self.y))]

    def kernel_amount(self):
        return {"qgemv_2bit": _gemv2_bytes(self.N, self.K, self.n_out, self.B)}

    def step_amount(self):
        return self.kernel_amount()["qgemv_2bit"]

    def config(self):
        return {"workload": self.name, "N": self.N, "K": self.K, "batch": self.B,
                "anchors": self.n_out, "formats": ["2bit_g32"], "rotate_copies": self.R}

    def cpu_baseline(self):
        import oracle
        idx = oracle.select_outliers(self.Wh, self.Xp, 0.035)
        rows = self.ORACLE_ROWS or self.N
        r = oracle.quantize_2bit(self.Wh[:rows], idx)
        c2 = oracle.pack_2bit(r["q"])
        what = "full" if rows == self.N else f"first {rows} rows of"
        return _time_oracle(
            lambda: oracle.gemv_2bit_ref(self.xh, oracle.unpack_2bit(c2), r["S"], r["Z"], r["idx"], r["W_O"]),
            _gemv2_bytes(rows, self.K, self.n_out, self.B), f"{what} {self.N}x{self.K} steps, batch {self.B}")


class Down70b(Decode14b):
    """The down projection of a 70B-shaped decoder (8192 x 28672, 3.5%
    anchors): at batch 8 its x does not fit one workgroup whole, so the call
    runs as K parts (grouped launches plus the in-order reduction)."""
    N, K = 8192, 28672
    SEED, PREFIX = 6, "down70b"
    ORACLE_ROWS = 512


class Decode14bInt4(Workload):
    """The v3.2 INT4 format at the 14B decode shape: channel permutation from
    a spiked calibration profile, the top 1% channels as fp16 anchors."""
    N, K = 13824, 5120

    def __init__(self, B):
        import torch
        from bit_weight_quantized_qw_amd import inputs, qw
        self.qw, self.B = qw, B
        self.name = f"decode14b_int4_b{B}"
        self.Wh = inputs.weight(self.N, self.K, workload=3)
        self.Xp = inputs.profile(256, self.K, workload=3)
        Wd = torch.from_numpy(self.Wh).cuda()
        perm = qw.qw_select_perm(Wd, torch.from_numpy(self.Xp).cuda())
        self.n_out = qw.qw_outlier_count(self.K, 0.01)
        p = qw.qw_pack_int4(Wd, perm, self.n_out)
        del Wd
        self.R = max(2, math.ceil(ROTATE_BYTES / p.nbytes()))
        self.p = _copies(p, self.R)
        x = torch.from_numpy(inputs.act_f16(B, self.K, workload=3).view(np.int16)).cuda().view(torch.float16)
        self.x = qw.qw_permute_cols(x, perm)
        self.perm_h = perm.cpu().numpy()
        self.y = torch.empty((B, self.N), dtype=torch.float16, device="cuda")

    def launches(self, i):
        r = i % self.R
        return [("qgemv_int4", lambda: self.qw.qgemv_int4(self.p[r], self.x, out=self.y))]

    def kernel_amount(self):
        return {"qgemv_int4": _int4_bytes(self.N, self.K, self.n_out, self.B)}

    def step_amount(self):
        return self.kernel_amount()["qgemv_int4"]

    def config(self):
        return {"workload": self.name, "N": self.N, "K": self.K, "batch": self.B, "anchors": self.n_out,
                "formats": ["int4_g32_perm"], "rotate_copies": self.R}

    def cpu_baseline(self):
        import oracle
        from bit_weight_quantized_qw_amd import inputs
        r = oracle.quantize_int4(self.Wh, self.perm_h, self.n_out)
        c = oracle.pack_int4(r["q"])
        x_p = oracle.permute_cols(inputs.act_f16(self.B, self.K, workload=3), self.perm_h)
        return _time_oracle(lambda: oracle.gemv_int4_ref(x_p, oracle.unpack_int4(c), r["s"], r["W_O"]),
                            self.step_amount(), f"full {self.N}x{self.K} steps, batch {self.B}")


class Decode32bStack(Workload):
    """64 layers x {qkv (grouped), o, gate/up with the gated activation,
    down}, batch 1. One token is 256 launches against distinct per-layer
    weights. The gate and up projections are one merged 55296 x 5120 matrix
    whose launch writes silu(gate) * up, and the down projection reads that
    output (the MLP half of each layer is chained as in decoding); q/k/v, o
    and gate/up read fixed per-layer inputs (attention is not part of the
    library)."""
    name = "decode32b_stack"
    steps, warmup = 50, 5
    L, H, I, KV = 64, 5120, 27648, 1024
    # (name, N, K, profile/input index); "gateup" is the merged gate/up matrix
    PROJ = [("q", 5120, 5120, 0), ("k", 1024, 5120, 0), ("v", 1024, 5120, 0),
            ("o", 5120, 5120, 1), ("gateup", 55296, 5120, 2), ("down", 5120, 27648, 3)]

    def __init__(self, layers=None):
        import torch
        from bit_weight_quantized_qw_amd import inputs, qw
        self.qw = qw
        self.L = layers or self.L
        self.w = []   # per layer: dict proj -> PackedWeight
        self.bytes_by_stage = {"qkv": 0, "o": 0, "gateup": 0, "down": 0}
        t0 = time.time()
        for l in range(self.L):
            prof = {}
            d = {}
            for p, (nm, N, K, inp) in enumerate(self.PROJ):
                if inp not in prof:
                    prof[inp] = inputs.torch_profile(256, K, workload=4, layer=l, proj=inp)
                W = inputs.torch_weight(N, K, workload=4, layer=l, proj=p)
                idx = qw.qw_select_outliers(W, prof[inp], 0.035)
                d[nm] = qw.qw_pack(W, qw.QW_FMT_2BIT_G32, idx)
                del W
            self.w.append(d)
            if l == 0:
                log(f"stack: layer 0 packed in {time.time() - t0:.1f}s")
        torch.cuda.synchronize()
        log(f"stack: {self.L} layers packed in {time.time() - t0:.1f}s")
        g = torch.Generator(device="cuda")
        g.manual_seed(inputs.torch_seed(4, 0, 0, inputs.ROLE_X))
        self.xs = [torch.randn((4, 1, max(self.H, self.I)), generator=g, device="cuda").half()
                   for _ in range(self.L)]
        self.yq = torch.empty((1, 5120), dtype=torch.float16, device="cuda")
        self.yk = torch.empty((1, 1024), dtype=torch.float16, device="cuda")
        self.yv = torch.empty((1, 1024), dtype=torch.float16, device="cuda")
        self.yo = torch.empty((1, 5120), dtype=torch.float16, device="cuda")
        self.yact = torch.empty((1, 27648), dtype=torch.float16, device="cuda")  # silu(gate) * up
        self.yd = torch.empty((1, 5120), dtype=torch.float16, device="cuda")

    def launches(self, i):
        qw = self.qw
        out = []
        for l in range(self.L):
            d, x = self.w[l], self.xs[l]
            out += [
                ("qkv", lambda d=d, x=x: qw.qgemv_2bit_grouped([d["q"], d["k"], d["v"]], x[0][:, :self.H],
                                                               outs=[self.yq, self.yk, self.yv])),
                ("o", lambda d=d, x=x: qw.qgemv_2bit(d["o"], x[1][:, :self.H], out=self.yo)),
                ("gateup", lambda d=d, x=x: qw.qgemv_2bit_swiglu(d["gateup"], x[2][:, :self.H], out=self.yact)),
                ("down", lambda d=d: qw.qgemv_2bit(d["down"], self.yact, out=self.yd)),
            ]
        return out

    def kernel_amount(self):
        b = {}
        d = self.w[0]
        nb = lambda p: _gemv2_bytes(p.N, p.K, p.n_out, 1)
        b["qkv"] = nb(d["q"]) + nb(d["k"]) + nb(d["v"]) - 2 * 2 * 5120
        b["o"] = nb(d["o"])
        b["gateup"] = nb(d["gateup"]) - self.I * 2  # I outputs, not 2I
        b["down"] = nb(d["down"])
        return b

    def step_amount(self):
        return self.L * sum(self.kernel_amount().values())

    def config(self):
        return {"workload": self.name, "layers": self.L, "hidden": self.H, "intermediate": self.I,
                "heads": "40q/8kv x 128", "batch": 1, "anchor_frac": 0.035,
                "formats": ["2bit_g32"], "mlp": "merged gate/up GEMV writes silu(gate)*up; down reads it",
                "launches_per_token": 4 * self.L}

    def cpu_baseline(self):
        import oracle
        from bit_weight_quantized_qw_amd import inputs
        frac_rows = 8
        jobs, amount = [], 0
        for p, (nm, N, K, inp) in enumerate(self.PROJ):
            W = inputs.weight(N, K, workload=4, layer=0, proj=p)
            X = inputs.profile(256, K, workload=4, layer=0, proj=inp)
            idx = oracle.select_outliers(W, X, 0.035)
            rows = N // frac_rows
            sel = np.arange(rows)
            if nm == "gateup":  # gate rows and the up rows they pair with
                sel = np.concatenate([np.arange(rows // 2), N // 2 + np.arange(rows // 2)])
            r = oracle.quantize_2bit(W[sel], idx)
            x = inputs.act_f16(1, K, workload=4, layer=0, proj=p)
            jobs.append((nm == "gateup", x, oracle.pack_2bit(r["q"]), r))
            amount += _gemv2_bytes(rows, K, len(idx), 1)

        def one():
            for sw, x, c, r in jobs:
                f = oracle.gemv_2bit_swiglu_ref if sw else oracle.gemv_2bit_ref
                f(x, oracle.unpack_2bit(c), r["S"], r["Z"], r["idx"], r["W_O"])
        return _time_oracle(one, amount, "layer 0, 1/8 of the rows of each of the 6 matrices "
                                         "(gate/up: the first 1/16 of each half, with the activation)")


class Decode32bStackFused(Decode32bStack):
    """The same token (same weights, inputs, the 448 products and the gated
    activation) as one persistent launch: the 256 stages run in order with a
    device-wide barrier between consecutive stages (qw_stack_run)."""
    name = "decode32b_stack_fused"
    graph = False  # one launch per token already

    def __init__(self, layers=None):
        super().__init__(layers)
        qw = self.qw
        self.ybuf = {}
        stages = []
        for l in range(self.L):
            d, x = self.w[l], self.xs[l]
            stages += [
                ([d["q"], d["k"], d["v"]], x[0][0, :self.H], [self.yq[0], self.yk[0], self.yv[0]]),
                ([d["o"]], x[1][0, :self.H], [self.yo[0]]),
                ([d["gateup"]], x[2][0, :self.H], [self.yact[0]], True),
                ([d["down"]], self.yact[0], [self.yd[0]]),
            ]
        self.stack = qw.Stack(stages)
        log(f"stack: {len(stages)} stages planned, {self.stack.handle.lds} B LDS per workgroup")

    def launches(self, i):
        return [("stack", self.stack.run)]

    def kernel_amount(self):
        return {"stack": self.L * sum(Decode32bStack.kernel_amount(self).values())}

    def step_amount(self):
        return self.kernel_amount()["stack"]

    def config(self):
        c = super().config()
        c["workload"] = self.name
        c["launches_per_token"] = 1
        return c


class Prefill70b(Workload):
    steps, warmup = 40, 5
    M, N, K = 2048, 28672, 8192
    unit = "TFLOP/s"
    bound = "mfma"
    dtype = "bf16"

    def __init__(self, fmt):
        import torch
        from bit_weight_quantized_qw_amd import inputs, qw
        self.qw = qw
        self.fmt = fmt
        self.name = "prefill70b_" + {qw.QW_FMT_NF4_B64: "nf4", qw.QW_FMT_2BIT_G32: "2bit",
                                     qw.QW_FMT_INT4_G32: "int4"}[fmt]
        W = inputs.torch_weight(self.N, self.K, workload=5)
        Xb = inputs.act_bf16_bits(self.M, self.K, workload=5)
        self.X = torch.from_numpy(Xb.view(np.int16)).cuda().view(torch.bfloat16)
        if fmt == qw.QW_FMT_INT4_G32:  # a fixed seeded permutation, no anchors
            self.perm_h = np.random.default_rng(5).permutation(self.K).astype(np.int32)
            perm = torch.from_numpy(self.perm_h).cuda()
            self.p = qw.qw_pack_int4(W, perm, 0)
            self.X = qw.qw_permute_cols(self.X, perm)
        else:
            self.p = qw.qw_pack(W, fmt)
        del W
        self.Y = torch.empty((self.M, self.N), dtype=torch.bfloat16, device="cuda")
        # the oracle's input: X in the order the kernel takes it
        self.Xb = Xb[:, self.perm_h] if fmt == qw.QW_FMT_INT4_G32 else Xb

    def launches(self, i):
        return [("qgemm_prefill", lambda: self.qw.qgemm_prefill(self.p, self.X, out=self.Y))]

    def kernel_amount(self):
        return {"qgemm_prefill": 2.0 * self.M * self.N * self.K}

    def kernel_bytes(self):  # X, the packed weight and Y, each once
        z = self.qw.qw_packed_sizes(self.fmt, self.N, self.K, 0)
        return {"qgemm_prefill": self.M * self.K * 2 + z["codes"] + z["scales"] + self.M * self.N * 2}

    def step_amount(self):
        return 2.0 * self.M * self.N * self.K

    def config(self):
        return {"workload": self.name, "M": self.M, "N": self.N, "K": self.K,
                "formats": [self.name.split("_")[1]], "out": "bf16"}

    def cpu_baseline(self):
        import oracle
        from bit_weight_quantized_qw_amd import inputs
        # bounded sample: 512 rows of W against all 2048 rows of X
        rows = 512
        W = inputs.weight(rows, self.K, workload=5, proj=1)
        if self.fmt == self.qw.QW_FMT_NF4_B64:
            q, a = oracle.quantize_nf4(W)
            c = oracle.pack_nf4(q)
            wb = lambda: oracle.prefill_weight_bf16_nf4(oracle.unpack_nf4(c), a)
        elif self.fmt == self.qw.QW_FMT_INT4_G32:
            r = oracle.quantize_int4(W, self.perm_h, 0)
            c = oracle.pack_int4(r["q"])
            wb = lambda: oracle.prefill_weight_bf16_int4(oracle.unpack_int4(c), r["s"], r["W_O"])
        else:
            r = oracle.quantize_2bit(W)
            c = oracle.pack_2bit(r["q"])
            wb = lambda: oracle.prefill_weight_bf16_2bit(oracle.unpack_2bit(c), r["S"], r["Z"])
        return _time_oracle(lambda: oracle.gemm_prefill_ref(self.Xb, wb()),
                            2.0 * self.M * rows * self.K,
                            f"2048x8192 X times a 512x8192 slice of W (fp64)", scale=1e12)


# fp64 operations per group of 32 in the 2-bit packer, counted from its
# formulas: single pass (mean, deviations, variance, squared deviations, the
# fit's sums, S and Z) 360; a refinement round (4 levels, 4 distances and 3
# minimum steps per weight, the refit) 429.
PACK2_FLOPS_PASS, PACK2_FLOPS_ROUND = 360, 429


class PrepLlama7b(Workload):
    """Device-side weight preparation of one 11008x4096 projection from fp16
    weights: profile sums, anchor selection, refined 2-bit pack."""
    name = "prep_llama7b_refine5"
    steps, warmup = 20, 3
    N, K, P, ROUNDS = 11008, 4096, 256, 5
    graph = False  # a preparation step, timed as issued once per weight
    bound = "alu"
    dtype = "f64"

    def __init__(self):
        import torch
        from bit_weight_quantized_qw_amd import inputs, qw
        self.qw = qw
        self.Wh = inputs.weight(self.N, self.K, workload=2).astype(np.float16)
        self.Xh = inputs.profile(self.P, self.K, workload=2).astype(np.float16)
        self.W = torch.from_numpy(self.Wh.view(np.int16)).cuda().view(torch.float16)
        self.X = torch.from_numpy(self.Xh.view(np.int16)).cuda().view(torch.float16)
        self.acc = torch.zeros(self.K, dtype=torch.float64, device="cuda")
        self.n_out = qw.qw_outlier_count(self.K, 0.035)
        self.idx = None

    def _select(self):
        self.idx = self.qw.qw_select_outliers_ex(self.W, self.acc, self.P, 0.035)

    def launches(self, i):
        return [("qw_profile_accumulate", lambda: (self.acc.zero_(), self.qw.qw_profile_accumulate(self.X, self.acc))),
                ("qw_select_outliers_ex", self._select),
                ("qw_pack_ex", lambda: self.qw.qw_pack_ex(self.W, self.qw.QW_FMT_2BIT_G32, self.idx,
                                                          refine_rounds=self.ROUNDS))]

    def kernel_amount(self):  # fp16 bytes each call consumes
        wb = self.N * self.K * 2
        return {"qw_profile_accumulate": self.P * self.K * 2, "qw_select_outliers_ex": wb, "qw_pack_ex": wb}

    def roof_amount(self):  # fp64 operations of the packer per call
        groups = self.N * self.K // 32
        return {"qw_pack_ex": groups * (PACK2_FLOPS_PASS + self.ROUNDS * PACK2_FLOPS_ROUND)}

    def step_amount(self):
        return self.N * self.K * 2

    def config(self):
        return {"workload": self.name, "N": self.N, "K": self.K, "weights": "fp16",
                "profile_rows": self.P, "anchors": self.n_out, "refine_rounds": self.ROUNDS}

    def cpu_baseline(self):
        import oracle
        rows = 512
        W32 = self.Wh[:rows].astype(np.float32)
        X32 = self.Xh.astype(np.float32)

        def one():
            idx = oracle.select_outliers(W32, X32, 0.035)
            oracle.quantize_2bit(W32, idx, refine_rounds=self.ROUNDS)
        return _time_oracle(one, rows * self.K * 2, f"{rows} of the {self.N} rows (profile, selection, 5-round pack)")


class CopyCalib(Workload):
    name = "copy_calib"
    library = False  # a torch kernel: timed with events recorded around it
    graph = False

    def __init__(self):
        import torch
        self.a = torch.empty(ROTATE_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        self.b = torch.empty_like(self.a)

    def launches(self, i):
        import torch
        return [("copy", lambda: torch.mul(self.a, 1.0, out=self.b))]

    def kernel_amount(self):
        return {"copy": 2 * ROTATE_BYTES}

    def step_amount(self):
        return 2 * ROTATE_BYTES

    def config(self):
        return {"workload": self.name, "bytes_read": ROTATE_BYTES, "bytes_written": ROTATE_BYTES}


def _time_oracle(fn, amount, sample, budget_s=12.0, scale=1e9):
    """Time the oracle's product path: >= 1 call, until budget_s elapsed."""
    try:
        from threadpoolctl import threadpool_limits
        cores = len(os.sched_getaffinity(0))
        ctx = threadpool_limits(limits=cores)
    except Exception:
        cores, ctx = 1, None
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    if ctx is not None:
        ctx.unregister() if hasattr(ctx, "unregister") else None
    return {"value": round(amount * n / dt / scale, 4), "cores": cores, "kind": "oracle",
            "sample": f"{n} x {sample}", "seconds": round(dt, 2)}


def _traffic(path, workload, kernel):
    """Counter-derived HBM bytes per launch, or None when there is no entry
    or the kernel's sources changed since the counters were taken."""
    import hashlib
    try:
        e = json.load(open(path))[workload][kernel]
        h = hashlib.sha256()
        for f in e["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        return e["bytes"] if h.hexdigest() == e["sha256"] else None
    except (OSError, KeyError, ValueError, TypeError):
        return None


WORKLOADS = {
    "llama7b_mlp_up_gemv": Llama7bMlpUp,
    "single_layer_2048": SingleLayer2048,
    "decode14b_b1": lambda: Decode14b(1), "decode14b_b2": lambda: Decode14b(2),
    "decode14b_b4": lambda: Decode14b(4), "decode14b_b8": lambda: Decode14b(8),
    "down70b_b1": lambda: Down70b(1), "down70b_b8": lambda: Down70b(8),
    "decode32b_stack": Decode32bStack,
    "decode32b_stack_fused": Decode32bStackFused,
    "decode14b_int4_b1": lambda: Decode14bInt4(1), "decode14b_int4_b8": lambda: Decode14bInt4(8),
    "prefill70b_nf4": lambda: Prefill70b(2), "prefill70b_2bit": lambda: Prefill70b(1),
    "prefill70b_int4": lambda: Prefill70b(3),
    "prep_llama7b_refine5": PrepLlama7b,
    "copy_calib": CopyCalib,
}


# --------------------------------------------------------------------- timing

def _sleep_rate():
    """GPU sleep cycles per ms (torch.cuda._sleep), measured once."""
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    s.record()
    torch.cuda._sleep(2_000_000)
    e.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(s.elapsed_time(e), 1e-3)


def run(wl, steps, warmup):
    """Returns (ms of the K timed steps, {kernel: [ms per launch]}, wall ms)."""
    import ctypes
    import torch
    from bit_weight_quantized_qw_amd import qw
    L = qw.lib()
    for i in range(warmup):
        for _, f in wl.launches(i):
            f()
    torch.cuda.synchronize()
    # per-launch kernel events (the library attaches them to its own
    # dispatches, so each pair brackets the kernel's execution only)
    plan = [wl.launches(warmup + i) for i in range(steps)]
    pairs = []
    for step in plan:
        for name, _ in step:
            s_ev = torch.cuda.Event(enable_timing=True)
            e_ev = torch.cuda.Event(enable_timing=True)
            pairs.append((name, s_ev, e_ev, qw._event_handle(s_ev), qw._event_handle(e_ev)))
    torch.cuda.synchronize()
    # host enqueue cost, to size the sleep that keeps the device queue full
    t0 = time.perf_counter()
    for i in range(warmup):
        for _, f in wl.launches(i):
            if wl.library:
                L.qw_time_next_call(pairs[0][3], pairs[0][4])
            f()
    torch.cuda.synchronize()
    per_step = (time.perf_counter() - t0) / max(warmup, 1)
    rate = _sleep_rate()
    sleep_ms = min(30000.0, 1.5 * per_step * steps * 1e3 + 5.0)

    first = torch.cuda.Event(enable_timing=True)
    last = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    torch.cuda._sleep(int(rate * sleep_ms))
    first.record()
    j = 0
    for step in plan:
        for _, f in step:
            _, s_ev, e_ev, hs, he = pairs[j]
            if wl.library:
                L.qw_time_next_call(hs, he)
                f()
            else:
                s_ev.record()
                f()
                e_ev.record()
            j += 1
    last.record()
    torch.cuda.synchronize()
    t_wall1 = time.perf_counter()
    total_ms = first.elapsed_time(last)
    per_kernel = {}
    for name, s_ev, e_ev, _, _ in pairs:
        per_kernel.setdefault(name, []).append(s_ev.elapsed_time(e_ev))
    wall_ms = (t_wall1 - t_wall0) * 1e3
    if wl.graph:
        total_ms, wall_ms = run_graph(wl, steps)
    return total_ms, per_kernel, wall_ms


def run_graph(wl, steps, max_nodes=2048):
    """Whole-step time of exactly K steps as HIP graph replays
    (torch.cuda.CUDAGraph on ROCm): C consecutive steps (the largest divisor
    of K whose launches stay within max_nodes) are captured once, with their
    own weight copies, and replayed K / C times, as a decode loop would run
    them. Returns (ms of the K steps, wall ms)."""
    import torch
    lps = max(1, len(wl.launches(0)))
    c = max(d for d in range(1, steps + 1) if steps % d == 0 and (d * lps <= max_nodes or d == 1))
    seq = [f for i in range(c) for _, f in wl.launches(i)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in seq:  # warm the captured sequence once eagerly
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in seq:
            f()
    g.replay()
    torch.cuda.synchronize()
    first = torch.cuda.Event(enable_timing=True)
    last = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    first.record()
    for _ in range(steps // c):
        g.replay()
    last.record()
    torch.cuda.synchronize()
    return first.elapsed_time(last), (time.perf_counter() - t0) * 1e3


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: per workload)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default: per workload)")
    ap.add_argument("--workload", default="decode32b_stack", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="leave out the prefill object of the default workload's line")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    ap.add_argument("--tune", action="append", default=[], metavar="NAME=VALUE",
                    help="set a library test hook for A/B runs (qw_tuning.h), e.g. "
                         "GEMV2_PATH=1 for the vector-ALU 2-bit GEMV; repeatable")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(2)
    from bit_weight_quantized_qw_amd import qw
    qw.lib()  # fail loudly if libqw.so is missing
    tuned = {}
    for t in args.tune:
        name, _, val = t.partition("=")
        key = getattr(qw, "QW_TUNE_" + name.upper(), None)
        if key is None or not val.lstrip("-").isdigit():
            print(f"unknown --tune {t}", file=sys.stderr)
            sys.exit(2)
        qw.qw_tune_set(key, int(val))
        tuned[name.upper()] = int(val)

    wl = WORKLOADS[args.workload]()
    log(f"workload {wl.name}: setup done")
    steps = args.steps if args.steps is not None else wl.steps
    warmup = args.warmup if args.warmup is not None else wl.warmup
    torch.cuda.synchronize()
    out = measure(wl, steps, warmup, args.traffic_json)
    if tuned:
        out["tune"] = tuned
    log(f"workload {wl.name}: {out['ms_per_step']} ms per step")
    if wl.name == "decode32b_stack" and not args.no_prefill:
        # the other half of the metric, timed in the same run
        pf = Prefill70b(1)
        log(f"workload {pf.name}: setup done")
        torch.cuda.synchronize()
        p = measure(pf, min(pf.steps, steps), min(pf.warmup, warmup), args.traffic_json)
        out["prefill"] = {k: p[k] for k in ("value", "unit", "steps", "warmup", "ms_per_step", "dtype",
                                           "config", "roofline", "kernels", "step_timing")}
        log(f"workload {pf.name}: {p['ms_per_step']} ms per call")
    if not args.no_cpu_baseline:
        cb = wl.cpu_baseline()
        if cb is not None:
            cb["unit"] = wl.unit
            out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


def measure(wl, steps, warmup, traffic_json):
    """Times one workload; returns the fields of the JSON line."""
    total_ms, per_kernel, wall_ms = run(wl, steps, warmup)
    ms_per_step = total_ms / steps
    scale = 1e12 if wl.unit == "TFLOP/s" else 1e9
    value = wl.step_amount() / (ms_per_step * 1e-3) / scale

    amounts = wl.kernel_amount()
    kbytes = wl.kernel_bytes()
    kstats = {}
    for nm, ds in per_kernel.items():
        avg = float(np.mean(ds))
        kstats[nm] = {"avg_us": round(avg * 1e3, 3), "launches": len(ds),
                      "achieved": round(amounts[nm] / (avg * 1e-3) / scale, 2),
                      "amount": int(amounts[nm])}  # algorithmic bytes (flops) per launch
        if nm in kbytes and kbytes[nm] != amounts[nm]:
            kstats[nm]["bytes"] = int(kbytes[nm])  # algorithmic bytes of a flop-bound launch
    dominant = max(kstats, key=lambda k: kstats[k]["avg_us"] * kstats[k]["launches"])
    peak = BF16_PEAK_TFLOPS if wl.bound == "mfma" else HBM_PEAK_GBS
    ach = kstats[dominant]["achieved"]
    roof_unit = wl.unit
    if wl.bound == "alu" and dominant in wl.roof_amount():  # fp64 operations per launch / time
        peak, roof_unit = FP64_PEAK_TFLOPS, "TFLOP/s"
        avg_s = kstats[dominant]["avg_us"] * 1e-6
        ach = round(wl.roof_amount()[dominant] / avg_s / 1e12, 3)
    traffic = _traffic(traffic_json, wl.name, dominant)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": wl.unit, "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded N(0,0.02^2) weights, N(0,1) activations)",
        "config": wl.config(),
        "roofline": {"bound": wl.bound, "kernel": dominant, "achieved": ach, "peak": peak,
                     "unit": roof_unit, "frac": round(ach / peak, 4), "traffic": traffic},
        "kernels": kstats,
        "wall_ms_timed_region": round(wall_ms, 3),
    }
    if wl.graph:
        out["step_timing"] = "hip graph replays of captured steps (kernel times: eager pass)"
    if wl.name.startswith("decode32b_stack"):
        out["tokens_per_s"] = round(1e3 / ms_per_step, 2)
    if hasattr(wl, "stack"):
        out["barrier_timeouts"] = wl.stack.error()
    return out


if __name__ == "__main__":
    main()
