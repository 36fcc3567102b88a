"""ctypes binding of libtiledattn.so (argument marshalling only).

Every step of attention runs in the HIP kernels behind the C ABI declared in
``include/tiledattn.h``; this module only checks tensor metadata, allocates
the outputs with torch (device memory is torch's job here) and passes raw
pointers and the current HIP stream.  There is no fallback: if the library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

LIB_NAME = "libtiledattn.so"
_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

TA_OK, TA_ERR_INVALID_ARG, TA_ERR_UNSUPPORTED, TA_ERR_MISALIGNED, TA_ERR_HIP = range(5)


def library_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Load (once) and return the HIP library; raise if it was never built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError("%s is not built; run __graft_entry__.build() (hipcc, gfx950)" % path)
        lib = ctypes.CDLL(path)
        lib.attn_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.attn_fwd.restype = ctypes.c_int
        lib.attn_status_string.argtypes = [ctypes.c_int]
        lib.attn_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
                 N: int, d: int, scale: float, causal: int, stream: int = 0) -> int:
    """Call the C entry point with raw addresses; returns the ta_status code."""
    return load_library().attn_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, N, d,
                                   ctypes.c_float(scale), causal, stream)


def attn_fwd(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None,
             stream=None):
    """Fused attention forward on the GPU.

    q, k, v: CUDA/HIP bfloat16 tensors [B, H, N, d], contiguous, same device.
    Returns (o float32 [B, H, N, d], lse float32 [B, H, N]); ``out``/``lse`` may
    be given to write into existing buffers.  ``scale`` defaults to 1/sqrt(d).
    """
    import torch
    lib = load_library()
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("q, k, v must be bfloat16")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one shape [B, H, N, d]")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = (int(x) for x in q.shape)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != (B, H, N, d) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 [B, H, N, d]")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, H, N, d, ctypes.c_float(float(scale)), int(bool(causal)), int(stream))
    if st != TA_OK:
        raise RuntimeError("attn_fwd failed: %s (status %d)" % (attn_status_string(st), st))
    return out, lse
