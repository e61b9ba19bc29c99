"""Thin ctypes binding over libqw.so (C ABI in include/qw.h).

Argument marshalling only: every step of quantization, packing and the
products runs in the library's HIP kernels. Torch tensors supply device
memory and the current stream. The functions carry the C names; the
``PackedWeight`` holder owns the torch buffers one packed matrix needs.

If libqw.so is missing this module raises on first use; there is no
fallback path.
"""

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqw.so")

QW_OK, QW_ERR_INVALID_ARG, QW_ERR_ALIGNMENT, QW_ERR_UNSUPPORTED, QW_ERR_HIP, QW_ERR_NO_DEVICE = range(6)
QW_ERR_SCRATCH_LIMIT = 6
QW_STATIC_SCRATCH_BYTES = 8 << 20
QW_FMT_2BIT_G32, QW_FMT_NF4_B64, QW_FMT_INT4_G32 = 1, 2, 3
QW_DT_F16, QW_DT_BF16, QW_DT_F32 = 1, 2, 3
QW_SCORE_MEANABS, QW_SCORE_L2 = 1, 2

# every function declared in include/qw.h and include/qw_tuning.h
EXPORTS = [
    "qw_abi_version", "qw_status_str", "qw_time_next_call", "qw_packed_sizes", "qw_outlier_count",
    "qw_codebook_2bit", "qw_nf4_levels", "qw_select_workspace_bytes", "qw_select_outliers",
    "qw_select_perm", "qw_permute_cols", "qw_pack",
    "qw_pack_ex", "qw_profile_accumulate", "qw_select_outliers_ex",
    "qw_stack_plan_bytes", "qw_stack_prepare", "qw_stack_sync_bytes", "qw_stack_run",
    "qgemv_2bit", "qgemv_2bit_workspace_bytes", "qgemv_2bit_ws", "qgemv_2bit_static", "qgemv_nf4", "qgemv_int4",
    "qgemv_2bit_grouped", "qgemv_2bit_swiglu",
    "qgemm_prefill", "qw_tune_set", "qw_tune_get",
]

# test hooks (include/qw_tuning.h)
QW_TUNE_GEMV2_PATH, QW_TUNE_GEMV2_SPLIT, QW_TUNE_GEMV2_DEEP_RING = 1, 2, 3
QW_TUNE_NF4_DEEP_RING, QW_TUNE_PREFILL_WIDE_TILES, QW_TUNE_INT4_PATH = 4, 5, 6
QW_TUNE_AUTO = -1


class QwError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {qw_status_str(status)} (status {status})")


class qw_weight(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
        ("n_out", ctypes.c_int32), ("n_out_pad", ctypes.c_int32),
        ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
        ("out_idx", ctypes.c_void_p), ("out_w", ctypes.c_void_p),
        ("out_mask", ctypes.c_void_p),
    ]


class qw_sizes(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_size_t), ("scales", ctypes.c_size_t), ("out_idx", ctypes.c_size_t),
        ("out_w", ctypes.c_size_t), ("out_mask", ctypes.c_size_t), ("n_out_pad", ctypes.c_int32),
    ]


class qw_stack_stage(ctypes.Structure):
    _fields_ = [
        ("count", ctypes.c_int32), ("w", qw_weight * 4), ("x", ctypes.c_void_p),
        ("y", ctypes.c_void_p * 4), ("y_dtype", ctypes.c_int32), ("swiglu", ctypes.c_int32),
    ]


class qw_stack(ctypes.Structure):
    _fields_ = [
        ("plan", ctypes.c_void_p), ("n_stages", ctypes.c_int32), ("grid", ctypes.c_int32),
        ("lds", ctypes.c_int32),
    ]


_lib = None


def lib():
    """Load libqw.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m bit_weight_quantized_qw_amd.build`")
    # torch ships its own HIP runtime: load it first, so libqw binds to that
    # same runtime (loaded the other way round, the process would hold two
    # runtimes and the library would see no current device)
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    c_i, c_d, c_p, c_sz = ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t
    W = ctypes.POINTER(qw_weight)
    sig = {
        "qw_abi_version": (c_i, []),
        "qw_status_str": (ctypes.c_char_p, [c_i]),
        "qw_time_next_call": (c_i, [c_p, c_p]),
        "qw_packed_sizes": (c_i, [c_i, c_i, c_i, c_i, ctypes.POINTER(qw_sizes)]),
        "qw_outlier_count": (c_i, [c_i, c_d]),
        "qw_codebook_2bit": (c_i, [ctypes.POINTER(ctypes.c_float)]),
        "qw_nf4_levels": (c_i, [ctypes.POINTER(ctypes.c_float)]),
        "qw_select_workspace_bytes": (c_sz, [c_i]),
        "qw_select_outliers": (c_i, [c_p, c_i, c_i, c_p, c_i, c_d, c_i, c_p, c_p, c_sz, c_p]),
        "qw_select_perm": (c_i, [c_p, c_i, c_i, c_p, c_i, c_i, c_p, c_p, c_sz, c_p]),
        "qw_permute_cols": (c_i, [c_p, c_i, c_i, c_i, c_p, c_p, c_p]),
        "qw_pack": (c_i, [c_p, W, c_p]),
        "qw_pack_ex": (c_i, [c_p, c_i, c_i, W, c_p]),
        "qw_profile_accumulate": (c_i, [c_p, c_i, c_i, c_i, c_p, c_p]),
        "qw_select_outliers_ex": (c_i, [c_p, c_i, c_i, c_i, c_p, ctypes.c_longlong, c_d, c_i, c_p, c_p,
                                        c_sz, c_p]),
        "qw_stack_plan_bytes": (c_sz, [c_i]),
        "qw_stack_prepare": (c_i, [ctypes.POINTER(qw_stack_stage), c_i, c_p, ctypes.POINTER(qw_stack)]),
        "qw_stack_sync_bytes": (c_sz, [ctypes.POINTER(qw_stack)]),
        "qw_stack_run": (c_i, [ctypes.POINTER(qw_stack), c_p, c_p]),
        "qgemv_2bit": (c_i, [W, c_p, c_i, c_p, c_i, c_p]),
        "qgemv_2bit_workspace_bytes": (c_i, [W, c_i, ctypes.POINTER(c_sz)]),
        "qgemv_2bit_ws": (c_i, [W, c_p, c_i, c_p, c_i, c_p, c_sz, c_p]),
        "qgemv_2bit_static": (c_i, [W, c_p, c_i, c_p, c_i, c_p]),
        "qgemv_nf4": (c_i, [W, c_p, c_i, c_p, c_i, c_p]),
        "qgemv_int4": (c_i, [W, c_p, c_i, c_p, c_i, c_p]),
        "qgemv_2bit_grouped": (c_i, [W, c_i, c_p, c_i, ctypes.POINTER(c_p), c_i, c_p]),
        "qgemv_2bit_swiglu": (c_i, [W, c_p, c_i, c_p, c_i, c_p]),
        "qgemm_prefill": (c_i, [W, c_p, c_i, c_p, c_i, c_p]),
        "qw_tune_set": (c_i, [c_i, c_i]),
        "qw_tune_get": (c_i, [c_i]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status, where):
    if status != QW_OK:
        raise QwError(status, where)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


# ---------------------------------------------------------------- host calls

def qw_abi_version():
    return lib().qw_abi_version()


def qw_status_str(status):
    return lib().qw_status_str(int(status)).decode()


def _event_handle(ev):
    if ev is None:
        return ctypes.c_void_p(0)
    if not ev.cuda_event:  # torch creates the HIP event at its first record
        ev.record()
    return ctypes.c_void_p(ev.cuda_event)


def qw_time_next_call(start_event, stop_event):
    """Arm the next library call on this thread to record kernel start/stop
    into two torch.cuda.Event(enable_timing=True) objects (either may be None)."""
    _check(lib().qw_time_next_call(_event_handle(start_event), _event_handle(stop_event)),
           "qw_time_next_call")


def qw_packed_sizes(fmt, N, K, n_out=0):
    """Dict of buffer byte counts and the anchor row stride."""
    z = qw_sizes()
    _check(lib().qw_packed_sizes(fmt, N, K, n_out, ctypes.byref(z)), "qw_packed_sizes")
    return {"codes": z.codes, "scales": z.scales, "out_idx": z.out_idx, "out_w": z.out_w,
            "out_mask": z.out_mask, "n_out_pad": z.n_out_pad}


def qw_outlier_count(K, frac):
    return lib().qw_outlier_count(int(K), float(frac))


def qw_codebook_2bit():
    out = (ctypes.c_float * 4)()
    _check(lib().qw_codebook_2bit(out), "qw_codebook_2bit")
    return np.array(out[:], dtype=np.float32)


def qw_nf4_levels():
    out = (ctypes.c_float * 16)()
    _check(lib().qw_nf4_levels(out), "qw_nf4_levels")
    return np.array(out[:], dtype=np.float32)


def qw_tune_set(key, value):
    """Set a test hook of include/qw_tuning.h (QW_TUNE_AUTO restores the
    automatic choice)."""
    _check(lib().qw_tune_set(int(key), int(value)), "qw_tune_set")


def qw_tune_get(key):
    return int(lib().qw_tune_get(int(key)))


class tuned:
    """Context manager: ``with tuned(QW_TUNE_GEMV2_PATH, 0): ...`` sets a hook
    for the block and restores its previous value afterwards."""

    def __init__(self, key, value):
        self.key, self.value = key, value

    def __enter__(self):
        self.prev = qw_tune_get(self.key)
        qw_tune_set(self.key, self.value)
        return self

    def __exit__(self, *exc):
        qw_tune_set(self.key, self.prev)
        return False


def qw_select_workspace_bytes(K):
    return int(lib().qw_select_workspace_bytes(int(K)))


def _select_workspace(K, device):
    import torch
    nb = qw_select_workspace_bytes(K)
    return torch.empty(max(nb, 16), dtype=torch.uint8, device=device), nb


# -------------------------------------------------------------- packed weight

class PackedWeight:
    """Device buffers of one packed matrix (torch tensors, caller-owned).
    out_idx holds the anchor channels (2-bit) or the channel permutation
    (INT4); out_w the fp16 anchors; out_mask the 2-bit anchor bit mask."""

    def __init__(self, fmt, N, K, n_out=0, device="cuda"):
        import torch
        z = qw_packed_sizes(fmt, N, K, n_out)
        self.format, self.N, self.K, self.n_out, self.n_out_pad = fmt, N, K, n_out, z["n_out_pad"]
        self.codes = torch.empty(z["codes"], dtype=torch.uint8, device=device)
        self.scales = torch.empty(z["scales"], dtype=torch.uint8, device=device)
        self.out_idx = self.out_w = self.out_mask = None
        if z["out_idx"]:
            self.out_idx = torch.empty(z["out_idx"] // 4, dtype=torch.int32, device=device)
        if z["out_w"]:
            self.out_w = torch.empty(z["out_w"] // 2, dtype=torch.int16, device=device)
        if z["out_mask"]:
            self.out_mask = torch.empty(z["out_mask"] // 4, dtype=torch.int32, device=device)

    def view(self):
        p = lambda t: t.data_ptr() if t is not None else None
        return qw_weight(self.format, self.N, self.K, self.n_out, self.n_out_pad,
                         self.codes.data_ptr(), self.scales.data_ptr(),
                         p(self.out_idx), p(self.out_w), p(self.out_mask))

    def nbytes(self):
        n = self.codes.numel() + self.scales.numel()
        for t in (self.out_idx, self.out_w, self.out_mask):
            if t is not None:
                n += t.numel() * t.element_size()
        return n

    # host copies in the oracle's array shapes
    def host_codes(self):
        return self.codes.cpu().numpy().reshape(self.N, -1)

    def host_scales(self):
        a = self.scales.cpu().numpy()
        if self.format == QW_FMT_2BIT_G32:
            return a.view(np.float16).reshape(self.N, self.K // 32, 2)
        if self.format == QW_FMT_INT4_G32:
            return a.view(np.float16).reshape(self.N, self.K // 32)
        return a.view(np.float32).reshape(self.N, self.K // 64)

    def host_out_w(self):
        if not self.n_out:
            return np.zeros((self.N, 0), np.float16)
        return self.out_w.cpu().numpy().view(np.float16).reshape(self.N, self.n_out_pad)


def _need(t, dtype, name, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def qw_select_outliers(W, X_prof, frac, score=QW_SCORE_MEANABS):
    import torch
    _need(W, torch.float32, "W", 2)
    _need(X_prof, torch.float32, "X_prof", 2)
    N, K = W.shape
    n = qw_outlier_count(K, frac)
    if n < 0:
        raise ValueError("frac must be in [0, 1)")
    out = torch.empty(max(n, 1), dtype=torch.int32, device=W.device)
    ws, nb = _select_workspace(K, W.device)
    _check(lib().qw_select_outliers(_ptr(W), N, K, _ptr(X_prof), X_prof.shape[0], float(frac),
                                    int(score), _ptr(out), _ptr(ws), nb, _stream()), "qw_select_outliers")
    return out[:n]


def _w_dtype(t):
    import torch
    m = {torch.float32: QW_DT_F32, torch.float16: QW_DT_F16, torch.bfloat16: QW_DT_BF16}
    if t.dtype not in m:
        raise TypeError(f"weights/activations must be fp32, fp16 or bf16, got {t.dtype}")
    return m[t.dtype]


def _need_any(t, name, ndim):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    return _w_dtype(t)


def qw_pack(W, fmt=QW_FMT_2BIT_G32, out_idx=None):
    """Quantize and pack fp32 W (N, K) on the device; returns PackedWeight."""
    import torch
    _need(W, torch.float32, "W", 2)
    return qw_pack_ex(W, fmt, out_idx)


def qw_pack_ex(W, fmt=QW_FMT_2BIT_G32, out_idx=None, refine_rounds=0):
    """qw_pack for fp32, fp16 or bf16 W (N, K), with ``refine_rounds`` rounds
    of nearest-level reassignment and refit (2-bit); returns PackedWeight."""
    import torch
    dt = _need_any(W, "W", 2)
    if fmt == QW_FMT_INT4_G32:
        raise ValueError("the INT4 format takes a permutation: use qw_pack_int4")
    N, K = W.shape
    n_out = 0 if out_idx is None else int(out_idx.numel())
    pw = PackedWeight(fmt, N, K, n_out, device=W.device)
    if n_out:
        _need(out_idx, torch.int32, "out_idx", 1)
        ok = bool(((out_idx[1:] > out_idx[:-1]).all() & (out_idx[0] >= 0) & (out_idx[-1] < K)).item())
        if not ok:
            raise ValueError("out_idx must be strictly ascending channels in [0, K)")
        pw.out_idx.copy_(out_idx)
    v = pw.view()
    _check(lib().qw_pack_ex(_ptr(W), dt, int(refine_rounds), ctypes.byref(v), _stream()), "qw_pack_ex")
    return pw


def qw_pack_int4(W, perm, n_out, refine_rounds=0):
    """Quantize and pack W (N, K; fp32, fp16 or bf16, original channel order)
    into the INT4 format with channel permutation ``perm`` (int32 (K,) CUDA
    tensor) and the first ``n_out`` permuted channels as fp16 anchors."""
    import torch
    dt = _need_any(W, "W", 2)
    _need(perm, torch.int32, "perm", 1)
    N, K = W.shape
    if perm.numel() != K:
        raise ValueError("perm must have K entries")
    pw = PackedWeight(QW_FMT_INT4_G32, N, K, int(n_out), device=W.device)
    pw.out_idx.copy_(perm)
    v = pw.view()
    _check(lib().qw_pack_ex(_ptr(W), dt, int(refine_rounds), ctypes.byref(v), _stream()), "qw_pack_ex")
    return pw


def qw_select_perm(W, X_prof, score=QW_SCORE_MEANABS):
    """INT4 channel permutation: channels by descending outlier score."""
    import torch
    _need(W, torch.float32, "W", 2)
    _need(X_prof, torch.float32, "X_prof", 2)
    N, K = W.shape
    out = torch.empty(K, dtype=torch.int32, device=W.device)
    ws, nb = _select_workspace(K, W.device)
    _check(lib().qw_select_perm(_ptr(W), N, K, _ptr(X_prof), X_prof.shape[0], int(score), _ptr(out),
                                _ptr(ws), nb, _stream()), "qw_select_perm")
    return out


def qw_permute_cols(X, perm, out=None):
    """X_p[:, j] = X[:, perm[j]] for a (M, K) fp16/bf16/fp32 CUDA tensor."""
    import torch
    dt = _need_any(X, "X", 2)
    _need(perm, torch.int32, "perm", 1)
    M, K = X.shape
    if perm.numel() != K:
        raise ValueError("perm must have K entries")
    Xp = out if out is not None else torch.empty_like(X)
    _need(Xp, X.dtype, "out", 2)
    if tuple(Xp.shape) != (M, K):
        raise ValueError("out must have the shape of X")
    _check(lib().qw_permute_cols(_ptr(X), dt, M, K, _ptr(perm), _ptr(Xp), _stream()), "qw_permute_cols")
    return Xp


def qw_profile_accumulate(X, abs_sum):
    """abs_sum (float64 [K], device) += column sums of |X| (M, K) in row order."""
    import torch
    dt = _need_any(X, "X", 2)
    _need(abs_sum, torch.float64, "abs_sum", 1)
    M, K = X.shape
    if abs_sum.numel() != K:
        raise ValueError("abs_sum must have K entries")
    _check(lib().qw_profile_accumulate(_ptr(X), dt, M, K, _ptr(abs_sum), _stream()),
           "qw_profile_accumulate")
    return abs_sum


def qw_select_outliers_ex(W, prof_abs_sum, prof_rows, frac, score=QW_SCORE_MEANABS):
    """Anchor channels from accumulated profile sums (qw_profile_accumulate)."""
    import torch
    dt = _need_any(W, "W", 2)
    _need(prof_abs_sum, torch.float64, "prof_abs_sum", 1)
    N, K = W.shape
    n = qw_outlier_count(K, frac)
    if n < 0:
        raise ValueError("frac must be in [0, 1)")
    out = torch.empty(max(n, 1), dtype=torch.int32, device=W.device)
    ws, nb = _select_workspace(K, W.device)
    _check(lib().qw_select_outliers_ex(_ptr(W), dt, N, K, _ptr(prof_abs_sum), int(prof_rows),
                                       float(frac), int(score), _ptr(out), _ptr(ws), nb, _stream()),
           "qw_select_outliers_ex")
    return out[:n]


_OUT = {"f16": QW_DT_F16, "bf16": QW_DT_BF16, "f32": QW_DT_F32}


def _dt(torch_dtype):
    import torch
    m = {torch.float16: QW_DT_F16, torch.bfloat16: QW_DT_BF16, torch.float32: QW_DT_F32}
    return m[torch_dtype]


def _io_shapes(pw, x, outs):
    """x must be (B, K) of the weight's K and every output (B, N_i) contiguous
    on the device: the library reads and writes exactly those sizes."""
    import torch
    if x.shape[1] != pw.K:
        raise ValueError(f"x has {x.shape[1]} columns, the weight K = {pw.K}")
    for y, N in outs:
        if not isinstance(y, torch.Tensor) or not y.is_cuda or not y.is_contiguous():
            raise ValueError("outputs must be contiguous CUDA tensors")
        if tuple(y.shape) != (x.shape[0], N):
            raise ValueError(f"output shape {tuple(y.shape)}, expected {(x.shape[0], N)}")


def qgemv_2bit(pw, x, out_dtype=None, out=None):
    import torch
    _need(x, torch.float16, "x", 2)
    out_dtype = out_dtype or torch.float16
    B = x.shape[0]
    y = out if out is not None else torch.empty((B, pw.N), dtype=out_dtype, device=x.device)
    _io_shapes(pw, x, [(y, pw.N)])
    v = pw.view()
    _check(lib().qgemv_2bit(ctypes.byref(v), _ptr(x), B, _ptr(y), _dt(y.dtype), _stream()),
           "qgemv_2bit")
    return y


def qgemv_2bit_workspace_bytes(pw, B):
    """Workspace bytes qgemv_2bit_ws needs for this weight at batch B."""
    n = ctypes.c_size_t(0)
    v = pw.view()
    _check(lib().qgemv_2bit_workspace_bytes(ctypes.byref(v), int(B), ctypes.byref(n)),
           "qgemv_2bit_workspace_bytes")
    return int(n.value)


def gemv_workspace(pw, B, device="cuda"):
    """A device workspace sized for qgemv_2bit_ws(pw, x of B rows), or None
    when that call needs none."""
    import torch
    nb = qgemv_2bit_workspace_bytes(pw, B)
    return torch.empty(nb, dtype=torch.uint8, device=device) if nb else None


def qgemv_2bit_ws(pw, x, workspace, out_dtype=None, out=None):
    """qgemv_2bit with a caller-owned workspace (a uint8 CUDA tensor, or None)."""
    import torch
    _need(x, torch.float16, "x", 2)
    out_dtype = out_dtype or torch.float16
    B = x.shape[0]
    y = out if out is not None else torch.empty((B, pw.N), dtype=out_dtype, device=x.device)
    _io_shapes(pw, x, [(y, pw.N)])
    nb = 0
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace")
        nb = workspace.numel()
    v = pw.view()
    _check(lib().qgemv_2bit_ws(ctypes.byref(v), _ptr(x), B, _ptr(y), _dt(y.dtype), _ptr(workspace), nb,
                               _stream()), "qgemv_2bit_ws")
    return y


def qgemv_2bit_static(pw, x, out):
    """qgemv_2bit_ws with the library's static device scratch instead of a
    workspace: the call allocates nothing (``out`` must be given)."""
    import torch
    _need(x, torch.float16, "x", 2)
    _io_shapes(pw, x, [(out, pw.N)])
    v = pw.view()
    _check(lib().qgemv_2bit_static(ctypes.byref(v), _ptr(x), x.shape[0], _ptr(out), _dt(out.dtype), _stream()),
           "qgemv_2bit_static")
    return out


def qgemv_nf4(pw, x, out_dtype=None, out=None):
    import torch
    _need(x, torch.float16, "x", 2)
    out_dtype = out_dtype or torch.float16
    B = x.shape[0]
    y = out if out is not None else torch.empty((B, pw.N), dtype=out_dtype, device=x.device)
    _io_shapes(pw, x, [(y, pw.N)])
    v = pw.view()
    _check(lib().qgemv_nf4(ctypes.byref(v), _ptr(x), B, _ptr(y), _dt(y.dtype), _stream()),
           "qgemv_nf4")
    return y


def qgemv_int4(pw, x_p, out_dtype=None, out=None):
    """INT4 GEMV; x_p (B, K) fp16 in the weight's permuted channel order."""
    import torch
    _need(x_p, torch.float16, "x_p", 2)
    out_dtype = out_dtype or torch.float16
    B = x_p.shape[0]
    y = out if out is not None else torch.empty((B, pw.N), dtype=out_dtype, device=x_p.device)
    _io_shapes(pw, x_p, [(y, pw.N)])
    v = pw.view()
    _check(lib().qgemv_int4(ctypes.byref(v), _ptr(x_p), B, _ptr(y), _dt(y.dtype), _stream()), "qgemv_int4")
    return y


def qgemv_2bit_grouped(pws, x, out_dtype=None, outs=None):
    import torch
    _need(x, torch.float16, "x", 2)
    out_dtype = out_dtype or torch.float16
    B = x.shape[0]
    n = len(pws)
    ys = outs if outs is not None else [
        torch.empty((B, p.N), dtype=out_dtype, device=x.device) for p in pws]
    if len(ys) != n:
        raise ValueError("one output per weight")
    for p, y in zip(pws, ys):
        _io_shapes(p, x, [(y, p.N)])
    arr = (qw_weight * n)(*[p.view() for p in pws])
    yp = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    _check(lib().qgemv_2bit_grouped(arr, n, _ptr(x), B, yp, _dt(ys[0].dtype), _stream()),
           "qgemv_2bit_grouped")
    return ys


def qgemv_2bit_swiglu(pw, x, out_dtype=None, out=None):
    """silu(gate) * up for a merged gate/up weight (gate rows over up rows,
    N = 2I): y (B, I)."""
    import torch
    _need(x, torch.float16, "x", 2)
    if pw.N % 32:
        raise ValueError("a merged gate/up weight has N = 2I rows with I % 16 == 0")
    out_dtype = out_dtype or torch.float16
    B = x.shape[0]
    y = out if out is not None else torch.empty((B, pw.N // 2), dtype=out_dtype, device=x.device)
    _io_shapes(pw, x, [(y, pw.N // 2)])
    v = pw.view()
    _check(lib().qgemv_2bit_swiglu(ctypes.byref(v), _ptr(x), B, _ptr(y), _dt(y.dtype), _stream()),
           "qgemv_2bit_swiglu")
    return y


def qgemm_prefill(pw, X, out_dtype=None, out=None):
    import torch
    _need(X, torch.bfloat16, "X", 2)
    out_dtype = out_dtype or torch.bfloat16
    M = X.shape[0]
    Y = out if out is not None else torch.empty((M, pw.N), dtype=out_dtype, device=X.device)
    _io_shapes(pw, X, [(Y, pw.N)])
    v = pw.view()
    _check(lib().qgemm_prefill(ctypes.byref(v), _ptr(X), M, _ptr(Y), _dt(Y.dtype), _stream()),
           "qgemm_prefill")
    return Y


# ------------------------------------------------------------------ stack

def qw_stack_plan_bytes(n_stages):
    return int(lib().qw_stack_plan_bytes(int(n_stages)))


class Stack:
    """A prepared fused decode stack (qw_stack_prepare) and its device plan
    and sync buffers. ``stages`` is a list of (weights, x, ys) or (weights,
    x, ys, swiglu): up to four PackedWeight (2-bit) sharing the fp16 input x
    (K,) and their outputs ys ((N_i,) fp16 or fp32 tensors); with swiglu
    true, one merged gate/up weight (N = 2I) whose output ys[0] (I,) gets
    silu(gate) * up. The tensors are referenced, not copied: each run reads
    and writes them in place."""

    def __init__(self, stages):
        import torch
        n = len(stages)
        arr = (qw_stack_stage * n)()
        self._keep = []
        for i, st in enumerate(stages):
            ws, x, ys = st[:3]
            sw = bool(st[3]) if len(st) > 3 else False
            if not 1 <= len(ws) <= 4 or len(ys) != len(ws):
                raise ValueError("a stage has 1..4 weights and as many outputs")
            if sw and len(ws) != 1:
                raise ValueError("a swiglu stage has one merged gate/up weight")
            _need(x, torch.float16, "x", 1)
            dt = ys[0].dtype
            for pw, y in zip(ws, ys):
                _need(y, dt, "y", 1)
                if pw.K != x.numel() or (pw.N // 2 if sw else pw.N) != y.numel():
                    raise ValueError("stage buffers must hold K inputs and the outputs of each weight")
            arr[i].count = len(ws)
            for m, (pw, y) in enumerate(zip(ws, ys)):
                arr[i].w[m] = pw.view()
                arr[i].y[m] = y.data_ptr()
            arr[i].x = x.data_ptr()
            arr[i].y_dtype = QW_DT_F32 if dt == torch.float32 else QW_DT_F16
            arr[i].swiglu = 1 if sw else 0
            self._keep.append((ws, x, ys))
        nb = qw_stack_plan_bytes(n)
        if nb == 0:
            raise ValueError("too many stages")
        self.plan = torch.empty(nb, dtype=torch.uint8, device="cuda")
        self.handle = qw_stack()
        _check(lib().qw_stack_prepare(arr, n, _ptr(self.plan), ctypes.byref(self.handle)), "qw_stack_prepare")
        sb = int(lib().qw_stack_sync_bytes(ctypes.byref(self.handle)))
        self.sync = torch.zeros(sb // 4, dtype=torch.int32, device="cuda")

    def run(self):
        """Enqueue one run of every stage on the current stream."""
        _check(lib().qw_stack_run(ctypes.byref(self.handle), _ptr(self.sync), _stream()), "qw_stack_run")

    def error(self):
        """Non-zero when a barrier wait of the last run gave up (synchronizes)."""
        return int(self.sync[0].item())
