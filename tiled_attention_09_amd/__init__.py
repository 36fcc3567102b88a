"""Fused attention forward for AMD Instinct MI355X (gfx950).

``attn_fwd(q, k, v, scale=None, causal=False) -> (o, lse)`` runs the HIP
kernel of ``csrc/`` through the C ABI of ``include/tiledattn.h``
(``libtiledattn.so``).  PyTorch only supplies device memory and the stream.
"""
from ._lib import (TA_ERR_HIP, TA_ERR_INVALID_ARG, TA_ERR_MISALIGNED, TA_ERR_UNSUPPORTED, TA_OK,
                   attn_fwd, attn_fwd_raw, attn_status_string, library_path, load_library)

__all__ = ["attn_fwd", "attn_fwd_raw", "attn_status_string", "library_path", "load_library",
           "TA_OK", "TA_ERR_INVALID_ARG", "TA_ERR_UNSUPPORTED", "TA_ERR_MISALIGNED", "TA_ERR_HIP"]
