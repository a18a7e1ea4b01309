"""Quantized paged-attention decode for AMD Instinct MI355X (gfx950).

The compute path is a HIP shared library (``libuq.so``) with a C ABI declared in
``include/uq_paged.h``; :mod:`quantized_paged_attention_amd.uq` is a thin ctypes
binding over it that takes torch device tensors.
"""

__all__ = ["uq", "synth"]
