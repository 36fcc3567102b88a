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
        lib.attn_fwd_ex.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 7 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.attn_fwd_ex.restype = ctypes.c_int
        lib.attn_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.attn_bwd.restype = ctypes.c_int
        lib.attn_bwd_workspace_size.argtypes = [ctypes.c_int] * 3
        lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
        lib.attn_quantize_fp8.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [
            ctypes.c_void_p]
        lib.attn_quantize_fp8.restype = ctypes.c_int
        lib.attn_fwd_fp8.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.attn_fwd_fp8.restype = ctypes.c_int
        lib.attn_fwd_dropout.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
        lib.attn_fwd_dropout.restype = ctypes.c_int
        lib.attn_fwd_split_workspace_size.argtypes = [ctypes.c_int] * 5
        lib.attn_fwd_split_workspace_size.restype = ctypes.c_size_t
        lib.attn_fwd_split.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 7 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.attn_fwd_split.restype = ctypes.c_int
        lib.attn_bwd_ex.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 7 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.attn_bwd_ex.restype = ctypes.c_int
        lib.attn_bwd_dropout.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
        lib.attn_bwd_dropout.restype = ctypes.c_int
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


def _fwd_buffers(q, k, v, out, lse):
    """Checks of the square forward's inputs; returns (B, H, N, d, out, lse)."""
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("q, k, v must be bfloat16")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one shape [B, H, N, d]")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = (int(x) for x in q.shape)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != (B, H, N, d) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 [B, H, N, d]")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    return B, H, N, d, out, lse


def attn_fwd_dropout_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int,
                         H: int, N: int, d: int, scale: float, causal: int, seed: int, drop_t: int,
                         stream: int = 0) -> int:
    """Call the dropout forward's C entry point with raw addresses; returns the status."""
    return load_library().attn_fwd_dropout(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, N, d,
                                           ctypes.c_float(scale), causal, seed, drop_t, stream)


def attn_fwd_dropout(q, k, v, seed: int, drop_t: int, scale: float | None = None,
                     causal: bool = False, out=None, lse=None, stream=None):
    """Fused attention forward with dropout on the probabilities.

    Like ``attn_fwd``; each probability P[i, j] of head b*H + h is kept when
    its Philox-4x32-10 byte (key ``seed``) is >= ``drop_t`` (drop probability
    drop_t / 256, 0..255) and the output is scaled by 256 / (256 - drop_t).
    ``lse`` is the undropped log-normaliser.  Returns (o, lse).
    """
    import torch
    B, H, N, d, out, lse = _fwd_buffers(q, k, v, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = load_library().attn_fwd_dropout(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
        ctypes.c_float(float(scale)), int(bool(causal)), int(seed) & ((1 << 64) - 1), int(drop_t),
        int(stream))
    if st != TA_OK:
        raise RuntimeError("attn_fwd_dropout failed: %s (status %d)" % (attn_status_string(st), st))
    return out, lse


def attn_fwd_ex_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
                    Nq: int, Nk: int, d: int, dv: int, query_offset: int, scale: float,
                    causal: int, stream: int = 0) -> int:
    """Call the general-shape C entry point with raw addresses; returns the status."""
    return load_library().attn_fwd_ex(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Nq, Nk, d, dv,
                                      query_offset, ctypes.c_float(scale), causal, stream)


def attn_fwd_ex(q, k, v, scale: float | None = None, causal: bool = False, query_offset: int = 0,
                out=None, lse=None, stream=None):
    """Attention forward for general shapes on the GPU.

    q: bf16 [B, H, Nq, d]; k: bf16 [B, H, Nk, d]; v: bf16 [B, H, Nk, dv] (device,
    contiguous).  Queries sit at absolute positions query_offset + i (causal rule:
    key j visible iff j <= i + query_offset).  Returns (o float32 [B, H, Nq, dv],
    lse float32 [B, H, Nq]); rows that see no key get o = 0 and lse = -inf.
    """
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous bfloat16 device tensor [B, H, rows, width]"
                             % name)
    B, H, Nq, d = (int(x) for x in q.shape)
    if tuple(k.shape[:2]) != (B, H) or int(k.shape[3]) != d or tuple(v.shape[:3]) != tuple(k.shape[:3]):
        raise ValueError("k must be [B, H, Nk, d] and v [B, H, Nk, dv]")
    Nk, dv = int(k.shape[2]), int(v.shape[3])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Nq, dv), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if out.shape != (B, H, Nq, dv) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 [B, H, Nq, dv]")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, Nq]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         B, H, Nq, Nk, d, dv, int(query_offset), ctypes.c_float(float(scale)),
                         int(bool(causal)), int(stream))
    if st != TA_OK:
        raise RuntimeError("attn_fwd_ex failed: %s (status %d)" % (attn_status_string(st), st))
    return out, lse


def attn_fwd_split_workspace_size(B: int, H: int, Nq: int, Nk: int, dv: int) -> int:
    """Bytes of device workspace ``attn_fwd_split`` uses (0: it runs unsplit)."""
    return int(load_library().attn_fwd_split_workspace_size(B, H, Nq, Nk, dv))


def attn_fwd_split_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int,
                       H: int, Nq: int, Nk: int, d: int, dv: int, query_offset: int, scale: float,
                       causal: int, ws_ptr: int, ws_bytes: int, stream: int = 0) -> int:
    """Call the split-key forward's C entry point with raw addresses; returns the status."""
    return load_library().attn_fwd_split(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Nq, Nk, d, dv,
                                         query_offset, ctypes.c_float(scale), causal, ws_ptr,
                                         ws_bytes, stream)


def attn_fwd_split(q, k, v, scale: float | None = None, causal: bool = False,
                   query_offset: int = 0, out=None, lse=None, workspace=None, stream=None):
    """``attn_fwd_ex`` with the key range split over workgroups when the
    (head, query tile) grid is small (decoding over long contexts); the partial
    results are combined exactly by their log-normalisers.  ``workspace`` (a
    uint8 device tensor of ``attn_fwd_split_workspace_size`` bytes) is
    allocated here when not given.  Returns (o, lse)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous bfloat16 device tensor [B, H, rows, width]"
                             % name)
    B, H, Nq, d = (int(x) for x in q.shape)
    if tuple(k.shape[:2]) != (B, H) or int(k.shape[3]) != d or tuple(v.shape[:3]) != tuple(k.shape[:3]):
        raise ValueError("k must be [B, H, Nk, d] and v [B, H, Nk, dv]")
    Nk, dv = int(k.shape[2]), int(v.shape[3])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Nq, dv), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if out.shape != (B, H, Nq, dv) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 [B, H, Nq, dv]")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, Nq]")
    need = attn_fwd_split_workspace_size(B, H, Nq, Nk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = load_library().attn_fwd_split(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
        dv, int(query_offset), ctypes.c_float(float(scale)), int(bool(causal)), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), int(stream))
    if st != TA_OK:
        raise RuntimeError("attn_fwd_split failed: %s (status %d)" % (attn_status_string(st), st))
    return out, lse


def attn_bwd_workspace_size(B: int, H: int, N: int) -> int:
    """Bytes of device workspace ``attn_bwd`` needs (0 if the sizes are out of range)."""
    return int(load_library().attn_bwd_workspace_size(B, H, N))


def attn_bwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, do_ptr: int,
                 dq_ptr: int, dk_ptr: int, dv_ptr: int, ws_ptr: int, B: int, H: int, N: int,
                 d: int, scale: float, causal: int, stream: int = 0) -> int:
    """Call the C entry point with raw addresses; returns the ta_status code."""
    return load_library().attn_bwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr,
                                   dv_ptr, ws_ptr, B, H, N, d, ctypes.c_float(scale), causal,
                                   stream)


def _bwd_buffers(q, k, v, o, lse, do, workspace, grads):
    """Checks of the backward's inputs; returns (B, H, N, d, workspace, grads)."""
    import torch
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("do", do, torch.bfloat16),
                        ("o", o, torch.float32)):
        if not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
        if t.dtype != dt:
            raise ValueError("%s must be %s" % (name, dt))
        if t.dim() != 4 or t.shape != q.shape or not t.is_contiguous():
            raise ValueError("%s must be contiguous with q's shape [B, H, N, d]" % name)
    B, H, N, d = (int(x) for x in q.shape)
    if not lse.is_cuda or lse.dtype != torch.float32 or lse.shape != (B, H, N) \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 device tensor [B, H, N]")
    ws_bytes = attn_bwd_workspace_size(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    if workspace.numel() * workspace.element_size() < ws_bytes or not workspace.is_cuda:
        raise ValueError("workspace must be a device buffer of at least %d bytes" % ws_bytes)
    if grads is None:
        grads = tuple(torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
                      for _ in range(3))
    for t in grads:
        if t.shape != (B, H, N, d) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("grads must be contiguous float32 [B, H, N, d]")
    return B, H, N, d, workspace, grads


def attn_bwd(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False,
             workspace=None, grads=None, stream=None):
    """Gradients of ``attn_fwd`` on the GPU.

    q, k, v, do: bfloat16 [B, H, N, d]; o float32 [B, H, N, d] and lse float32
    [B, H, N] from ``attn_fwd`` with the same scale and causal flag.  Returns
    (dq, dk, dv), float32 [B, H, N, d].  ``workspace`` (a uint8 device tensor of
    at least ``attn_bwd_workspace_size`` bytes) and ``grads`` (three float32
    tensors) may be given to reuse buffers.
    """
    import torch
    lib = load_library()
    B, H, N, d, workspace, grads = _bwd_buffers(q, k, v, o, lse, do, workspace, grads)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    dq, dk, dv = grads
    st = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      workspace.data_ptr(), B, H, N, d, ctypes.c_float(float(scale)),
                      int(bool(causal)), int(stream))
    if st != TA_OK:
        raise RuntimeError("attn_bwd failed: %s (status %d)" % (attn_status_string(st), st))
    return dq, dk, dv


def attn_bwd_ex_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, do_ptr: int,
                    dq_ptr: int, dk_ptr: int, dv_ptr: int, ws_ptr: int, B: int, H: int, Nq: int,
                    Nk: int, d: int, dv: int, query_offset: int, scale: float, causal: int,
                    stream: int = 0) -> int:
    """Call the general-shape backward's C entry point with raw addresses; returns the status."""
    return load_library().attn_bwd_ex(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr,
                                      dv_ptr, ws_ptr, B, H, Nq, Nk, d, dv, query_offset,
                                      ctypes.c_float(scale), causal, stream)


def attn_bwd_ex(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False,
                query_offset: int = 0, workspace=None, grads=None, stream=None):
    """Gradients of ``attn_fwd_ex`` on the GPU (same scale, causal flag, offset).

    q, do: bf16 [B, H, Nq, d] and [B, H, Nq, dv]; k, v: bf16 [B, H, Nk, d],
    [B, H, Nk, dv]; o float32 [B, H, Nq, dv], lse float32 [B, H, Nq].  Returns
    (dq [B, H, Nq, d], dk [B, H, Nk, d], dv [B, H, Nk, dv]), float32.
    """
    import torch
    lib = load_library()
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("do", do, torch.bfloat16),
                        ("o", o, torch.float32), ("lse", lse, torch.float32)):
        if not t.is_cuda or t.dtype != dt or not t.is_contiguous():
            raise ValueError("%s must be a contiguous %s device tensor" % (name, dt))
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, rows, width]")
    B, H, Nq, d = (int(x) for x in q.shape)
    Nk, dvw = int(k.shape[2]), int(v.shape[3])
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape[:3]) != (B, H, Nk):
        raise ValueError("k must be [B, H, Nk, d] and v [B, H, Nk, dv]")
    if tuple(do.shape) != (B, H, Nq, dvw) or tuple(o.shape) != (B, H, Nq, dvw) \
            or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("do and o must be [B, H, Nq, dv], lse [B, H, Nq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = attn_bwd_workspace_size(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    if workspace.numel() * workspace.element_size() < ws_bytes or not workspace.is_cuda:
        raise ValueError("workspace must be a device buffer of at least %d bytes" % ws_bytes)
    shapes = ((B, H, Nq, d), (B, H, Nk, d), (B, H, Nk, dvw))
    if grads is None:
        grads = tuple(torch.empty(sh, dtype=torch.float32, device=q.device) for sh in shapes)
    for t, sh in zip(grads, shapes):
        if tuple(t.shape) != sh or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("grads must be contiguous float32 dq %s, dk %s, dv %s" % shapes)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    dq, dk, dv = grads
    st = lib.attn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                         workspace.data_ptr(), B, H, Nq, Nk, d, dvw, int(query_offset),
                         ctypes.c_float(float(scale)), int(bool(causal)), int(stream))
    if st != TA_OK:
        raise RuntimeError("attn_bwd_ex failed: %s (status %d)" % (attn_status_string(st), st))
    return dq, dk, dv


def attn_bwd_dropout_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                         do_ptr: int, dq_ptr: int, dk_ptr: int, dv_ptr: int, ws_ptr: int, B: int,
                         H: int, N: int, d: int, scale: float, causal: int, seed: int,
                         drop_t: int, stream: int = 0) -> int:
    """Call the dropout backward's C entry point with raw addresses; returns the status."""
    return load_library().attn_bwd_dropout(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr,
                                           dk_ptr, dv_ptr, ws_ptr, B, H, N, d,
                                           ctypes.c_float(scale), causal, seed, drop_t, stream)


def attn_bwd_dropout(q, k, v, o, lse, do, seed: int, drop_t: int, scale: float | None = None,
                     causal: bool = False, workspace=None, grads=None, stream=None):
    """Gradients of ``attn_fwd_dropout`` (same seed, drop_t, scale, causal): the
    mask is regenerated, never stored.  Arguments and results as ``attn_bwd``."""
    import torch
    lib = load_library()
    B, H, N, d, workspace, grads = _bwd_buffers(q, k, v, o, lse, do, workspace, grads)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    dq, dk, dv = grads
    st = lib.attn_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), workspace.data_ptr(), B, H, N, d,
                              ctypes.c_float(float(scale)), int(bool(causal)),
                              int(seed) & ((1 << 64) - 1), int(drop_t), int(stream))
    if st != TA_OK:
        raise RuntimeError("attn_bwd_dropout failed: %s (status %d)" % (attn_status_string(st), st))
    return dq, dk, dv


def attn_quantize_fp8(x, out=None, descale=None, stream=None):
    """Per-head FP8 (OCP E4M3) codes of a bf16 device tensor [..., rows, d].

    Returns (codes uint8 tensor of x's shape, descale float32 tensor of shape
    x.shape[:-2]) with x ~= e4m3(codes) * descale.
    """
    import torch
    lib = load_library()
    if not x.is_cuda or x.dtype != torch.bfloat16 or x.dim() < 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 device tensor [..., rows, d]")
    rows, d = int(x.shape[-2]), int(x.shape[-1])
    heads = x.numel() // max(rows * d, 1)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if descale is None:
        descale = torch.empty(x.shape[:-2], dtype=torch.float32, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = lib.attn_quantize_fp8(x.data_ptr(), out.data_ptr(), descale.data_ptr(), heads, rows, d,
                               int(stream))
    if st != TA_OK:
        raise RuntimeError("attn_quantize_fp8 failed: %s (status %d)" % (attn_status_string(st), st))
    return out, descale


def attn_fwd_fp8_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, qd_ptr, kd_ptr, B, H, N, d, scale,
                     causal, stream=0) -> int:
    return load_library().attn_fwd_fp8(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, qd_ptr, kd_ptr, B, H,
                                       N, d, ctypes.c_float(scale), causal, stream)


def attn_fwd_fp8(q8, k8, v, q_descale, k_descale, scale: float | None = None, causal=False,
                 out=None, lse=None, stream=None):
    """Attention forward with FP8 scores: q8, k8 uint8 E4M3 codes [B, H, N, d]
    (from attn_quantize_fp8), v bf16 [B, H, N, d], descales float32 [B, H]."""
    import torch
    lib = load_library()
    if q8.dtype != torch.uint8 or k8.dtype != torch.uint8 or v.dtype != torch.bfloat16:
        raise ValueError("q8, k8 must be uint8 codes and v bfloat16")
    if q8.dim() != 4 or q8.shape != k8.shape or q8.shape != v.shape:
        raise ValueError("q8, k8, v must share one shape [B, H, N, d]")
    for t in (q8, k8, v, q_descale, k_descale):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("inputs must be contiguous device tensors")
    B, H, N, d = (int(x) for x in q8.shape)
    if tuple(q_descale.shape) != (B, H) or tuple(k_descale.shape) != (B, H) \
            or q_descale.dtype != torch.float32 or k_descale.dtype != torch.float32:
        raise ValueError("descales must be float32 [B, H]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    if stream is None:
        stream = torch.cuda.current_stream(q8.device).cuda_stream
    st = lib.attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), q_descale.data_ptr(), k_descale.data_ptr(), B, H, N, d,
                          ctypes.c_float(float(scale)), int(bool(causal)), int(stream))
    if st != TA_OK:
        raise RuntimeError("attn_fwd_fp8 failed: %s (status %d)" % (attn_status_string(st), st))
    return out, lse
