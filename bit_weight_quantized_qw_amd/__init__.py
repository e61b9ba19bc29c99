"""MI355X (gfx950) fused low-bit dequant-GEMV / prefill-GEMM library.

The compute lives in ``libqw.so`` (hand-written HIP, C ABI declared in
``include/qw.h``). ``bit_weight_quantized_qw_amd.qw`` is a thin ctypes
binding over it; importing this package does not load the library, so the
CPU-only parts (``inputs``) stay importable on machines without a GPU.
"""

__all__ = ["inputs", "qw"]
