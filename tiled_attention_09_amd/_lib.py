"""ctypes binding of libtiledattn.so (argument marshalling only).

Every step of attention runs in the HIP kernels behind the C ABI declared in
``include/tiledattn.h``; this module only checks tensor metadata, allocates
the outputs with torch (device memory is torch's job here) and passes raw
pointers and the current HIP stream.  There is no fallback: if the library is
missing, every call raises.

Every tensor a caller passes -- inputs, outputs, workspaces -- is checked for
dtype, shape, contiguity and device before the C entry point is called: a
host tensor or a short buffer given as an output would otherwise be written
out of bounds by a kernel.
"""
from __future__ import annotations

import ctypes
import math
import os

LIB_NAME = "libtiledattn.so"
_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

(TA_OK, TA_ERR_INVALID_ARG, TA_ERR_UNSUPPORTED, TA_ERR_MISALIGNED, TA_ERR_HIP,
 TA_ERR_TOO_LARGE) = range(6)

_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

# name: (argument types, result type)
_SIGNATURES = {
    "attn_fwd": ([_P] * 5 + [_I] * 4 + [_F, _I, _P], _I),
    "attn_fwd_ex": ([_P] * 5 + [_I] * 7 + [_F, _I, _P], _I),
    "attn_bwd": ([_P] * 10 + [_I] * 4 + [_F, _I, _P], _I),
    "attn_bwd_workspace_size": ([_I] * 3, _Z),
    "attn_quantize_fp8": ([_P] * 3 + [_I] * 3 + [_P], _I),
    "attn_fwd_fp8": ([_P] * 7 + [_I] * 4 + [_F, _I, _P], _I),
    "attn_fwd_dropout": ([_P] * 5 + [_I] * 4 + [_F, _I, ctypes.c_uint64, _I, _P], _I),
    "attn_fwd_split_workspace_size": ([_I] * 5, _Z),
    "attn_fwd_split": ([_P] * 5 + [_I] * 7 + [_F, _I, _P, _Z, _P], _I),
    "attn_bwd_ex": ([_P] * 10 + [_I] * 7 + [_F, _I, _P], _I),
    "attn_bwd_dropout": ([_P] * 10 + [_I] * 4 + [_F, _I, ctypes.c_uint64, _I, _P], _I),
    "attn_bwd_noalloc": ([_P] * 9 + [_I] * 4 + [_F, _I, _P], _I),
    "attn_fwd_dropout_ex": ([_P] * 5 + [_I] * 7 + [_F, _I, ctypes.c_uint64, _I, _P], _I),
    "attn_bwd_dropout_ex": ([_P] * 10 + [_I] * 7 + [_F, _I, ctypes.c_uint64, _I, _P], _I),
    "attn_fwd_fp8_ex": ([_P] * 7 + [_I] * 7 + [_F, _I, _P], _I),
    "attn_status_string": ([_I], ctypes.c_char_p),
}


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
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _check(st: int, name: str) -> None:
    if st != TA_OK:
        raise RuntimeError("%s failed: %s (status %d)" % (name, attn_status_string(st), st))


# ---------------------------------------------------------------- argument checks

def _dev_input(t, name: str, dtype, dims: int | None = 4):
    """A caller's input: a contiguous device tensor of ``dtype`` with ``dims``
    dimensions (any number when None); raises ValueError otherwise."""
    if not getattr(t, "is_cuda", False):
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s" % (name, dtype))
    if dims is not None and t.dim() != dims:
        raise ValueError("%s must have %d dimensions" % (name, dims))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _same_device(ref, *named):
    """Every (name, tensor) pair in ``named`` lives on ref's device."""
    for name, t in named:
        if t.device != ref.device:
            raise ValueError("%s must be on %s (got %s)" % (name, ref.device, t.device))


def _dev_output(t, name: str, shape, dtype, device):
    """An output buffer: allocated on ``device`` when ``t`` is None, else checked
    for shape, dtype, contiguity and device."""
    import torch
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != shape or t.dtype != dtype or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s" % (name, dtype, list(shape)))
    if not getattr(t, "is_cuda", False) or t.device != device:
        raise ValueError("%s must be a device tensor on %s" % (name, device))
    return t


def _dev_workspace(t, name: str, need: int, device):
    """A byte workspace of at least ``need`` bytes on ``device`` (allocated when None)."""
    import torch
    if t is None:
        return torch.empty(max(int(need), 256), dtype=torch.uint8, device=device)
    if not getattr(t, "is_cuda", False) or t.device != device or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device buffer on %s" % (name, device))
    if t.numel() * t.element_size() < need:
        raise ValueError("%s must hold at least %d bytes" % (name, need))
    return t


def _stream(stream, device) -> int:
    """The caller's stream handle, or the current stream of ``device``."""
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream(device).cuda_stream)


def _scale(scale, d: int) -> ctypes.c_float:
    """The caller's scale, or 1/sqrt(d) (the lab's default)."""
    return ctypes.c_float(float(1.0 / math.sqrt(d) if scale is None else scale))


def _fwd_buffers(q, k, v, out, lse):
    """Checks of the square forward's tensors; returns (B, H, N, d, out, lse)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_input(t, name, torch.bfloat16)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one shape [B, H, N, d]")
    _same_device(q, ("k", k), ("v", v))
    B, H, N, d = (int(x) for x in q.shape)
    out = _dev_output(out, "out", (B, H, N, d), torch.float32, q.device)
    lse = _dev_output(lse, "lse", (B, H, N), torch.float32, q.device)
    return B, H, N, d, out, lse


def _ex_buffers(q, k, v, out, lse):
    """Checks of the general-shape forward's tensors; returns
    (B, H, Nq, Nk, d, dv, out, lse)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_input(t, name, torch.bfloat16)
    _same_device(q, ("k", k), ("v", v))
    B, H, Nq, d = (int(x) for x in q.shape)
    if tuple(k.shape[:2]) != (B, H) or int(k.shape[3]) != d or tuple(v.shape[:3]) != tuple(k.shape[:3]):
        raise ValueError("k must be [B, H, Nk, d] and v [B, H, Nk, dv]")
    Nk, dv = int(k.shape[2]), int(v.shape[3])
    out = _dev_output(out, "out", (B, H, Nq, dv), torch.float32, q.device)
    lse = _dev_output(lse, "lse", (B, H, Nq), torch.float32, q.device)
    return B, H, Nq, Nk, d, dv, out, lse


def _bwd_buffers(q, k, v, o, lse, do, workspace, grads):
    """Checks of the square backward's tensors; returns (B, H, N, d, workspace, grads)."""
    import torch
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("do", do, torch.bfloat16),
                        ("o", o, torch.float32)):
        _dev_input(t, name, dt)
        if t.shape != q.shape:
            raise ValueError("%s must have q's shape [B, H, N, d]" % name)
    _dev_input(lse, "lse", torch.float32, 3)
    _same_device(q, ("k", k), ("v", v), ("do", do), ("o", o), ("lse", lse))
    B, H, N, d = (int(x) for x in q.shape)
    if tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be [B, H, N]")
    if workspace is not _NO_WORKSPACE:
        workspace = _dev_workspace(workspace, "workspace", attn_bwd_workspace_size(B, H, N),
                                   q.device)
    grads = (None, None, None) if grads is None else tuple(grads)
    if len(grads) != 3:
        raise ValueError("grads must be three tensors (dq, dk, dv)")
    grads = tuple(_dev_output(t, n, (B, H, N, d), torch.float32, q.device)
                  for t, n in zip(grads, ("dq", "dk", "dv")))
    return B, H, N, d, workspace, grads


_NO_WORKSPACE = object()   # _bwd_buffers: the entry point takes no workspace


# ---------------------------------------------------------------- forward

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
    lib = load_library()
    B, H, N, d, out, lse = _fwd_buffers(q, k, v, out, lse)
    _check(lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H, N, d, _scale(scale, d), int(bool(causal)), _stream(stream, q.device)),
           "attn_fwd")
    return out, lse


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
    lib = load_library()
    B, H, N, d, out, lse = _fwd_buffers(q, k, v, out, lse)
    _check(lib.attn_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, H, N, d, _scale(scale, d), int(bool(causal)),
                                int(seed) & ((1 << 64) - 1), int(drop_t), _stream(stream, q.device)),
           "attn_fwd_dropout")
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
    lib = load_library()
    B, H, Nq, Nk, d, dv, out, lse = _ex_buffers(q, k, v, out, lse)
    _check(lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           B, H, Nq, Nk, d, dv, int(query_offset), _scale(scale, d),
                           int(bool(causal)), _stream(stream, q.device)),
           "attn_fwd_ex")
    return out, lse


def attn_fwd_dropout_ex(q, k, v, seed: int, drop_t: int, scale: float | None = None,
                        causal: bool = False, query_offset: int = 0, out=None, lse=None,
                        stream=None):
    """``attn_fwd_ex`` with the dropout of ``attn_fwd_dropout``; query row r of
    the chunk draws the mask row of its absolute position query_offset + r.
    Returns (o, lse)."""
    lib = load_library()
    B, H, Nq, Nk, d, dv, out, lse = _ex_buffers(q, k, v, out, lse)
    _check(lib.attn_fwd_dropout_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, Nq, Nk, d, dv, int(query_offset),
                                   _scale(scale, d), int(bool(causal)),
                                   int(seed) & ((1 << 64) - 1), int(drop_t),
                                   _stream(stream, q.device)),
           "attn_fwd_dropout_ex")
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
    lib = load_library()
    B, H, Nq, Nk, d, dv, out, lse = _ex_buffers(q, k, v, out, lse)
    need = attn_fwd_split_workspace_size(B, H, Nq, Nk, dv)
    workspace = _dev_workspace(workspace, "workspace", need, q.device)
    _check(lib.attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, H, Nq, Nk, d, dv, int(query_offset),
                              _scale(scale, d), int(bool(causal)), workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(),
                              _stream(stream, q.device)),
           "attn_fwd_split")
    return out, lse


# ---------------------------------------------------------------- backward

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


def attn_bwd(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False,
             workspace=None, grads=None, stream=None):
    """Gradients of ``attn_fwd`` on the GPU.

    q, k, v, do: bfloat16 [B, H, N, d]; o float32 [B, H, N, d] and lse float32
    [B, H, N] from ``attn_fwd`` with the same scale and causal flag.  Returns
    (dq, dk, dv), float32 [B, H, N, d].  ``workspace`` (a uint8 device tensor of
    at least ``attn_bwd_workspace_size`` bytes) and ``grads`` (three float32
    tensors) may be given to reuse buffers.
    """
    lib = load_library()
    B, H, N, d, workspace, (dq, dk, dv) = _bwd_buffers(q, k, v, o, lse, do, workspace, grads)
    _check(lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                        workspace.data_ptr(), B, H, N, d, _scale(scale, d), int(bool(causal)),
                        _stream(stream, q.device)),
           "attn_bwd")
    return dq, dk, dv


def attn_bwd_ex_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, do_ptr: int,
                    dq_ptr: int, dk_ptr: int, dv_ptr: int, ws_ptr: int, B: int, H: int, Nq: int,
                    Nk: int, d: int, dv: int, query_offset: int, scale: float, causal: int,
                    stream: int = 0) -> int:
    """Call the general-shape backward's C entry point with raw addresses; returns the status."""
    return load_library().attn_bwd_ex(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr,
                                      dv_ptr, ws_ptr, B, H, Nq, Nk, d, dv, query_offset,
                                      ctypes.c_float(scale), causal, stream)


def _bwd_ex_buffers(q, k, v, o, lse, do, workspace, grads):
    """Checks of the general-shape backward's tensors; returns
    (B, H, Nq, Nk, d, dv, workspace, (dq, dk, dv))."""
    import torch
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("do", do, torch.bfloat16),
                        ("o", o, torch.float32)):
        _dev_input(t, name, dt)
    _dev_input(lse, "lse", torch.float32, 3)
    _same_device(q, ("k", k), ("v", v), ("do", do), ("o", o), ("lse", lse))
    B, H, Nq, d = (int(x) for x in q.shape)
    Nk, dvw = int(k.shape[2]), int(v.shape[3])
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape[:3]) != (B, H, Nk):
        raise ValueError("k must be [B, H, Nk, d] and v [B, H, Nk, dv]")
    if tuple(do.shape) != (B, H, Nq, dvw) or tuple(o.shape) != (B, H, Nq, dvw) \
            or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("do and o must be [B, H, Nq, dv], lse [B, H, Nq]")
    workspace = _dev_workspace(workspace, "workspace", attn_bwd_workspace_size(B, H, Nq), q.device)
    shapes = ((B, H, Nq, d), (B, H, Nk, d), (B, H, Nk, dvw))
    grads = (None, None, None) if grads is None else tuple(grads)
    if len(grads) != 3:
        raise ValueError("grads must be three tensors (dq, dk, dv)")
    grads = tuple(_dev_output(t, n, sh, torch.float32, q.device)
                  for t, n, sh in zip(grads, ("dq", "dk", "dv"), shapes))
    return B, H, Nq, Nk, d, dvw, workspace, grads


def attn_bwd_ex(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False,
                query_offset: int = 0, workspace=None, grads=None, stream=None):
    """Gradients of ``attn_fwd_ex`` on the GPU (same scale, causal flag, offset).

    q, do: bf16 [B, H, Nq, d] and [B, H, Nq, dv]; k, v: bf16 [B, H, Nk, d],
    [B, H, Nk, dv]; o float32 [B, H, Nq, dv], lse float32 [B, H, Nq].  Returns
    (dq [B, H, Nq, d], dk [B, H, Nk, d], dv [B, H, Nk, dv]), float32.
    """
    lib = load_library()
    B, H, Nq, Nk, d, dvw, workspace, (dq, dk, dv) = _bwd_ex_buffers(q, k, v, o, lse, do,
                                                                    workspace, grads)
    _check(lib.attn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                           workspace.data_ptr(), B, H, Nq, Nk, d, dvw, int(query_offset),
                           _scale(scale, d), int(bool(causal)), _stream(stream, q.device)),
           "attn_bwd_ex")
    return dq, dk, dv


def attn_bwd_dropout_ex(q, k, v, o, lse, do, seed: int, drop_t: int, scale: float | None = None,
                        causal: bool = False, query_offset: int = 0, workspace=None, grads=None,
                        stream=None):
    """Gradients of ``attn_fwd_dropout_ex`` (same shapes, offset, seed and drop_t);
    arguments and results as ``attn_bwd_ex``."""
    lib = load_library()
    B, H, Nq, Nk, d, dvw, workspace, (dq, dk, dv) = _bwd_ex_buffers(q, k, v, o, lse, do,
                                                                    workspace, grads)
    _check(lib.attn_bwd_dropout_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), workspace.data_ptr(), B, H, Nq, Nk, d, dvw,
                                   int(query_offset), _scale(scale, d), int(bool(causal)),
                                   int(seed) & ((1 << 64) - 1), int(drop_t),
                                   _stream(stream, q.device)),
           "attn_bwd_dropout_ex")
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
    lib = load_library()
    B, H, N, d, workspace, (dq, dk, dv) = _bwd_buffers(q, k, v, o, lse, do, workspace, grads)
    _check(lib.attn_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), workspace.data_ptr(), B, H, N, d, _scale(scale, d),
                                int(bool(causal)), int(seed) & ((1 << 64) - 1), int(drop_t),
                                _stream(stream, q.device)),
           "attn_bwd_dropout")
    return dq, dk, dv


def attn_bwd_noalloc_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                         do_ptr: int, dq_ptr: int, dk_ptr: int, dv_ptr: int, B: int, H: int,
                         N: int, d: int, scale: float, causal: int, stream: int = 0) -> int:
    """Call the no-allocation backward's C entry point with raw addresses; returns the status."""
    return load_library().attn_bwd_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr,
                                           dk_ptr, dv_ptr, B, H, N, d, ctypes.c_float(scale),
                                           causal, stream)


def attn_bwd_noalloc(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False,
                     grads=None, stream=None):
    """``attn_bwd`` without a workspace: the library keeps the row statistics in
    its own fixed device scratch (16 MiB per device, B*H*N <= 2^21), so a caller
    that passes ``grads`` allocates nothing.  Calls that may overlap on one
    device race on that scratch.  Returns (dq, dk, dv)."""
    lib = load_library()
    B, H, N, d, _, (dq, dk, dv) = _bwd_buffers(q, k, v, o, lse, do, _NO_WORKSPACE, grads)
    _check(lib.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), B, H, N, d, _scale(scale, d), int(bool(causal)),
                                _stream(stream, q.device)),
           "attn_bwd_noalloc")
    return dq, dk, dv


# ---------------------------------------------------------------- FP8 scores

def attn_quantize_fp8(x, out=None, descale=None, stream=None):
    """Per-head FP8 (OCP E4M3) codes of a bf16 device tensor [..., rows, d].

    Returns (codes uint8 tensor of x's shape, descale float32 tensor of shape
    x.shape[:-2]) with x ~= e4m3(codes) * descale.
    """
    import torch
    lib = load_library()
    _dev_input(x, "x", torch.bfloat16, None)
    if x.dim() < 2:
        raise ValueError("x must be [..., rows, d]")
    rows, d = int(x.shape[-2]), int(x.shape[-1])
    heads = x.numel() // max(rows * d, 1)
    out = _dev_output(out, "out", x.shape, torch.uint8, x.device)
    descale = _dev_output(descale, "descale", x.shape[:-2], torch.float32, x.device)
    _check(lib.attn_quantize_fp8(x.data_ptr(), out.data_ptr(), descale.data_ptr(), heads, rows, d,
                                 _stream(stream, x.device)),
           "attn_quantize_fp8")
    return out, descale


def attn_fwd_fp8_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, qd_ptr, kd_ptr, B, H, N, d, scale,
                     causal, stream=0) -> int:
    """Call the FP8-score forward's C entry point with raw addresses; returns the status."""
    return load_library().attn_fwd_fp8(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, qd_ptr, kd_ptr, B, H,
                                       N, d, ctypes.c_float(scale), causal, stream)


def attn_fwd_fp8(q8, k8, v, q_descale, k_descale, scale: float | None = None, causal=False,
                 out=None, lse=None, stream=None):
    """Attention forward with FP8 scores: q8, k8 uint8 E4M3 codes [B, H, N, d]
    (from attn_quantize_fp8), v bf16 [B, H, N, d], descales float32 [B, H]
    (positive and finite, as attn_quantize_fp8 writes them)."""
    import torch
    lib = load_library()
    _dev_input(q8, "q8", torch.uint8)
    _dev_input(k8, "k8", torch.uint8)
    _dev_input(v, "v", torch.bfloat16)
    if q8.shape != k8.shape or q8.shape != v.shape:
        raise ValueError("q8, k8, v must share one shape [B, H, N, d]")
    B, H, N, d = (int(x) for x in q8.shape)
    _dev_input(q_descale, "q_descale", torch.float32, 2)
    _dev_input(k_descale, "k_descale", torch.float32, 2)
    if tuple(q_descale.shape) != (B, H) or tuple(k_descale.shape) != (B, H):
        raise ValueError("descales must be float32 [B, H]")
    _same_device(q8, ("k8", k8), ("v", v), ("q_descale", q_descale), ("k_descale", k_descale))
    out = _dev_output(out, "out", (B, H, N, d), torch.float32, q8.device)
    lse = _dev_output(lse, "lse", (B, H, N), torch.float32, q8.device)
    _check(lib.attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), q_descale.data_ptr(), k_descale.data_ptr(), B, H, N, d,
                            _scale(scale, d), int(bool(causal)), _stream(stream, q8.device)),
           "attn_fwd_fp8")
    return out, lse


def attn_fwd_fp8_ex(q8, k8, v, q_descale, k_descale, scale: float | None = None, causal=False,
                    query_offset: int = 0, out=None, lse=None, stream=None):
    """``attn_fwd_fp8`` for general shapes: q8 [B, H, Nq, d], k8 [B, H, Nk, d]
    E4M3 codes, v bf16 [B, H, Nk, dv], descales float32 [B, H]; query r at
    position query_offset + r.  Returns (o [B, H, Nq, dv], lse [B, H, Nq])."""
    import torch
    lib = load_library()
    _dev_input(q8, "q8", torch.uint8)
    _dev_input(k8, "k8", torch.uint8)
    _dev_input(v, "v", torch.bfloat16)
    B, H, Nq, d = (int(x) for x in q8.shape)
    if tuple(k8.shape[:2]) != (B, H) or int(k8.shape[3]) != d or tuple(v.shape[:3]) != tuple(k8.shape[:3]):
        raise ValueError("k8 must be [B, H, Nk, d] and v [B, H, Nk, dv]")
    Nk, dv = int(k8.shape[2]), int(v.shape[3])
    _dev_input(q_descale, "q_descale", torch.float32, 2)
    _dev_input(k_descale, "k_descale", torch.float32, 2)
    if tuple(q_descale.shape) != (B, H) or tuple(k_descale.shape) != (B, H):
        raise ValueError("descales must be float32 [B, H]")
    _same_device(q8, ("k8", k8), ("v", v), ("q_descale", q_descale), ("k_descale", k_descale))
    out = _dev_output(out, "out", (B, H, Nq, dv), torch.float32, q8.device)
    lse = _dev_output(lse, "lse", (B, H, Nq), torch.float32, q8.device)
    _check(lib.attn_fwd_fp8_ex(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), q_descale.data_ptr(), k_descale.data_ptr(), B, H,
                               Nq, Nk, d, dv, int(query_offset), _scale(scale, d),
                               int(bool(causal)), _stream(stream, q8.device)),
           "attn_fwd_fp8_ex")
    return out, lse
