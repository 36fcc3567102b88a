"""Fused attention forward and backward for AMD Instinct MI355X (gfx950).

``attn_fwd(q, k, v, scale=None, causal=False) -> (o, lse)``,
``attn_fwd_ex(q, k, v, scale, causal, query_offset)`` (Nq != Nk, dv != d) with
``attn_bwd_ex`` and ``attn_fwd_split`` (keys split over workgroups for decoding), and
``attn_bwd(q, k, v, o, lse, do, scale=None, causal=False) -> (dq, dk, dv)``,
``attn_fwd_fp8`` (FP8 scores) and ``attn_fwd_dropout`` / ``attn_bwd_dropout`` (reproducible dropout) run
the HIP kernels of ``csrc/`` through the C ABI of ``include/tiledattn.h``
(``libtiledattn.so``).  PyTorch only supplies device memory and the stream.
"""
from ._lib import (TA_ERR_HIP, TA_ERR_INVALID_ARG, TA_ERR_MISALIGNED, TA_ERR_TOO_LARGE,
                   TA_ERR_UNSUPPORTED, TA_OK,
                   attn_bwd, attn_bwd_dropout, attn_bwd_dropout_raw, attn_bwd_ex, attn_bwd_ex_raw,
                   attn_bwd_dropout_ex, attn_bwd_noalloc, attn_bwd_noalloc_raw, attn_bwd_raw,
                   attn_fwd_dropout_ex, attn_fwd_fp8_ex,
                   attn_bwd_workspace_size, attn_fwd, attn_fwd_ex,
                   attn_fwd_dropout, attn_fwd_dropout_raw, attn_fwd_ex_raw, attn_fwd_fp8,
                   attn_fwd_split, attn_fwd_split_raw, attn_fwd_split_workspace_size,
                   attn_fwd_fp8_raw, attn_fwd_raw,
                   attn_quantize_fp8,
                   attn_status_string, library_path, load_library)

__all__ = ["attn_fwd", "attn_fwd_raw", "attn_fwd_ex", "attn_fwd_ex_raw", "attn_fwd_fp8",
           "attn_fwd_fp8_raw", "attn_fwd_split", "attn_fwd_split_raw",
           "attn_fwd_split_workspace_size", "attn_fwd_dropout", "attn_fwd_dropout_ex", "attn_fwd_fp8_ex",
           "attn_bwd_dropout_ex", "attn_fwd_dropout_raw", "attn_quantize_fp8", "attn_bwd", "attn_bwd_raw", "attn_bwd_ex", "attn_bwd_ex_raw", "attn_bwd_dropout", "attn_bwd_dropout_raw", "attn_bwd_noalloc", "attn_bwd_noalloc_raw", "attn_bwd_workspace_size",
           "attn_status_string", "library_path", "load_library",
           "TA_OK", "TA_ERR_INVALID_ARG", "TA_ERR_UNSUPPORTED", "TA_ERR_MISALIGNED", "TA_ERR_HIP",
           "TA_ERR_TOO_LARGE"]
