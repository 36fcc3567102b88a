"""CPU tests of the C-ABI library: it loads, exports what the header declares,
and rejects bad arguments before any HIP call (so no GPU is needed)."""
from __future__ import annotations

import ctypes
import math
import os
import re
import subprocess

import pytest

import tiled_attention_09_amd as ta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tiledattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ta.library_path()),
                                reason="libtiledattn.so not built (run __graft_entry__.build())")


def _gpu_visible() -> bool:
    import torch
    return torch.cuda.device_count() > 0   # counts devices without initialising HIP


# The fake-address tests are host-logic tests: never run them where a GPU could
# execute a launch that slipped through a validation bug.
host_only = pytest.mark.skipif(_gpu_visible(), reason="fake-address checks run on hosts without a GPU")

# Fake, suitably aligned addresses: every call below must be rejected by the
# argument checks, so these are never dereferenced and no kernel is enqueued.
A = 0x100000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_entry_points():
    assert declared_functions() == ["attn_bwd", "attn_bwd_dropout", "attn_bwd_dropout_ex",
                                    "attn_bwd_ex",
                                    "attn_bwd_noalloc", "attn_bwd_workspace_size",
                                    "attn_fwd",
                                    "attn_fwd_dropout", "attn_fwd_dropout_ex", "attn_fwd_ex",
                                    "attn_fwd_fp8", "attn_fwd_fp8_ex",
                                    "attn_fwd_split", "attn_fwd_split_workspace_size",
                                    "attn_quantize_fp8", "attn_status_string"]


def test_library_exports_every_declared_symbol():
    lib = ta.load_library()
    out = subprocess.run(["nm", "-D", "--defined-only", ta.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings():
    for st in range(6):
        assert ta.attn_status_string(st)
    assert ta.attn_status_string(99) == "unknown status"
    assert "head dimension" in ta.attn_status_string(ta.TA_ERR_UNSUPPORTED)


def call(**over):
    args = dict(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, N=128, d=64, scale=0.125, causal=0)
    args.update(over)
    return ta.attn_fwd_raw(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                           args["H"], args["N"], args["d"], args["scale"], args["causal"], 0)


@host_only
@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_null_pointer(field):
    assert call(**{field: 0}) == ta.TA_ERR_INVALID_ARG


@host_only
@pytest.mark.parametrize("over", [dict(B=0), dict(H=0), dict(N=0), dict(B=-1), dict(N=(1 << 22) + 1),
                                  dict(causal=2), dict(causal=-1), dict(scale=math.inf),
                                  dict(scale=-math.inf), dict(scale=math.nan),
                                  dict(B=1 << 16, H=1 << 15, N=1 << 20)])
def test_invalid_sizes_flags_scale(over):
    assert call(**over) == ta.TA_ERR_INVALID_ARG


@host_only
@pytest.mark.parametrize("d", [0, 16, 32, 96, 100, 256])
def test_unsupported_head_dim(d):
    assert call(d=d) == ta.TA_ERR_UNSUPPORTED


@host_only
@pytest.mark.parametrize("field,val", [("q", A + 8), ("k", A + 2), ("v", A + 4), ("o", A + 8),
                                       ("lse", A + 2), ("lse", A + 1)])
def test_misaligned(field, val):
    # every other argument valid and d supported: the call must stop at the alignment check
    assert call(**{field: val}) == ta.TA_ERR_MISALIGNED


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ta.attn_fwd(x, x, x)


def test_ctypes_signature():
    lib = ta.load_library()
    assert lib.attn_fwd.restype is ctypes.c_int
    assert len(lib.attn_fwd.argtypes) == 12
    assert lib.attn_bwd.restype is ctypes.c_int
    assert len(lib.attn_bwd.argtypes) == 17


# ---- backward entry point -------------------------------------------------

BWD_PTRS = ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "ws"]


def call_bwd(**over):
    args = dict({p: A for p in BWD_PTRS}, B=1, H=1, N=128, d=64, scale=0.125, causal=0)
    args.update(over)
    return ta.attn_bwd_raw(*(args[p] for p in BWD_PTRS), args["B"], args["H"], args["N"],
                           args["d"], args["scale"], args["causal"], 0)


def test_workspace_size():
    assert ta.attn_bwd_workspace_size(2, 32, 8192) == 2 * 32 * 8192 * 8
    assert ta.attn_bwd_workspace_size(1, 1, 1003) == 1004 * 8    # rows padded to a multiple of 4
    assert ta.attn_bwd_workspace_size(1, 1, 1001) == 1004 * 8
    assert ta.attn_bwd_workspace_size(3, 5, 1) == 15 * 4 * 8
    assert ta.attn_bwd_workspace_size(0, 1, 8) == 0
    assert ta.attn_bwd_workspace_size(1, 1, (1 << 22) + 1) == 0


@host_only
@pytest.mark.parametrize("field", BWD_PTRS)
def test_bwd_null_pointer(field):
    assert call_bwd(**{field: 0}) == ta.TA_ERR_INVALID_ARG


@host_only
@pytest.mark.parametrize("over", [dict(B=0), dict(H=0), dict(N=0), dict(N=(1 << 22) + 1),
                                  dict(causal=2), dict(scale=math.nan), dict(scale=math.inf),
                                  dict(B=1 << 16, H=1 << 15, N=1 << 20)])
def test_bwd_invalid_sizes_flags_scale(over):
    assert call_bwd(**over) == ta.TA_ERR_INVALID_ARG


@host_only
@pytest.mark.parametrize("d", [0, 32, 96, 256])
def test_bwd_unsupported_head_dim(d):
    assert call_bwd(d=d) == ta.TA_ERR_UNSUPPORTED


@host_only
@pytest.mark.parametrize("field,off", [(p, 8) for p in BWD_PTRS if p != "lse"] + [("lse", 2)])
def test_bwd_misaligned(field, off):
    assert call_bwd(**{field: A + off}) == ta.TA_ERR_MISALIGNED


def test_python_bwd_wrapper_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    o = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        ta.attn_bwd(x, x, x, o, torch.zeros(1, 1, 8), x)


# ---- general-shape forward ---------------------------------------------------

def call_ex(**over):
    args = dict(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, Nq=16, Nk=128, d=64, dv=128, off=112,
                scale=0.125, causal=1)
    args.update(over)
    return ta.attn_fwd_ex_raw(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                              args["H"], args["Nq"], args["Nk"], args["d"], args["dv"], args["off"],
                              args["scale"], args["causal"], 0)


@host_only
@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_ex_null_pointer(field):
    assert call_ex(**{field: 0}) == ta.TA_ERR_INVALID_ARG


@host_only
@pytest.mark.parametrize("over", [dict(off=-1), dict(off=(1 << 30) + 1), dict(Nq=-1), dict(Nk=-1),
                                  dict(Nq=(1 << 22) + 1), dict(Nk=(1 << 22) + 1), dict(B=0),
                                  dict(causal=3), dict(scale=math.nan)])
def test_ex_invalid(over):
    assert call_ex(**over) == ta.TA_ERR_INVALID_ARG


@host_only
@pytest.mark.parametrize("d,dv", [(64, 32), (32, 64), (128, 256), (96, 128)])
def test_ex_unsupported_widths(d, dv):
    assert call_ex(d=d, dv=dv) == ta.TA_ERR_UNSUPPORTED


@host_only
@pytest.mark.parametrize("field,val", [("q", A + 8), ("v", A + 4), ("o", A + 8), ("lse", A + 2)])
def test_ex_misaligned(field, val):
    assert call_ex(**{field: val}) == ta.TA_ERR_MISALIGNED


@host_only
def test_ex_no_queries_is_a_no_op():
    # every argument valid; Nq = 0 returns before any HIP call, NULL allowed for empty tensors
    assert call_ex(Nq=0) == ta.TA_OK
    assert call_ex(Nq=0, q=0, o=0, lse=0) == ta.TA_OK


@host_only
@pytest.mark.parametrize("field", ["k", "v"])
def test_ex_null_keys_only_when_empty(field):
    assert call_ex(**{field: 0}) == ta.TA_ERR_INVALID_ARG


@host_only
def test_square_entry_rejects_empty():
    assert call(N=0) == ta.TA_ERR_INVALID_ARG


# ---- FP8 entry points -----------------------------------------------------------

FP8_PTRS = ["q", "k", "v", "o", "lse", "qd", "kd"]


def call_fp8(**over):
    args = dict({p: A for p in FP8_PTRS}, B=1, H=2, N=256, d=128, scale=0.09, causal=1)
    args.update(over)
    return ta.attn_fwd_fp8_raw(*(args[p] for p in FP8_PTRS), args["B"], args["H"], args["N"],
                               args["d"], args["scale"], args["causal"], 0)


@host_only
@pytest.mark.parametrize("field", FP8_PTRS)
def test_fp8_null_pointer(field):
    assert call_fp8(**{field: 0}) == ta.TA_ERR_INVALID_ARG


@host_only
@pytest.mark.parametrize("over", [dict(N=0), dict(B=0), dict(causal=5), dict(scale=math.inf)])
def test_fp8_invalid(over):
    assert call_fp8(**over) == ta.TA_ERR_INVALID_ARG


@host_only
@pytest.mark.parametrize("d", [32, 96, 256])
def test_fp8_head_dims(d):
    assert call_fp8(d=d) == ta.TA_ERR_UNSUPPORTED


@host_only
@pytest.mark.parametrize("field,off", [("q", 8), ("k", 4), ("v", 8), ("o", 8), ("lse", 2),
                                       ("qd", 2), ("kd", 1)])
def test_fp8_misaligned(field, off):
    assert call_fp8(**{field: A + off}) == ta.TA_ERR_MISALIGNED


@host_only
def test_quantize_validation():
    lib = ta.load_library()
    q = lambda x=A, o=A, dsc=A, heads=2, rows=16, d=64: lib.attn_quantize_fp8(x, o, dsc, heads, rows, d, 0)
    assert q(x=0) == ta.TA_ERR_INVALID_ARG
    assert q(heads=0) == ta.TA_ERR_INVALID_ARG
    assert q(rows=0) == ta.TA_ERR_INVALID_ARG
    assert q(d=96) == ta.TA_ERR_UNSUPPORTED
    assert q(o=A + 8) == ta.TA_ERR_MISALIGNED
    assert q(dsc=A + 2) == ta.TA_ERR_MISALIGNED


# ---- dropout entry points -------------------------------------------------------

def call_drop(**over):
    args = dict(q=A, k=A, v=A, o=A, lse=A, B=1, H=2, N=256, d=128, scale=0.09, causal=1,
                seed=12345, t=64)
    args.update(over)
    return ta.attn_fwd_dropout_raw(args["q"], args["k"], args["v"], args["o"], args["lse"],
                                   args["B"], args["H"], args["N"], args["d"], args["scale"],
                                   args["causal"], args["seed"], args["t"], 0)


@host_only
@pytest.mark.parametrize("over", [dict(q=0), dict(lse=0), dict(N=0), dict(B=0), dict(causal=2),
                                  dict(scale=math.nan), dict(t=-1), dict(t=256)])
def test_dropout_fwd_invalid(over):
    assert call_drop(**over) == ta.TA_ERR_INVALID_ARG


@host_only
def test_dropout_fwd_head_dims():
    assert call_drop(d=96) == ta.TA_ERR_UNSUPPORTED


@host_only
@pytest.mark.parametrize("field,off", [("q", 8), ("v", 4), ("o", 8), ("lse", 2)])
def test_dropout_fwd_misaligned(field, off):
    assert call_drop(**{field: A + off}) == ta.TA_ERR_MISALIGNED


BWD_PTRS = ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "ws"]


def call_bwd_drop(**over):
    args = dict({p: A for p in BWD_PTRS}, B=1, H=2, N=256, d=128, scale=0.09, causal=1,
                seed=7, t=26)
    args.update(over)
    return ta.attn_bwd_dropout_raw(*(args[p] for p in BWD_PTRS), args["B"], args["H"], args["N"],
                                   args["d"], args["scale"], args["causal"], args["seed"],
                                   args["t"], 0)


@host_only
@pytest.mark.parametrize("over", [dict(do=0), dict(ws=0), dict(N=0), dict(H=0), dict(causal=-1),
                                  dict(scale=math.inf), dict(t=-1), dict(t=300)])
def test_dropout_bwd_invalid(over):
    assert call_bwd_drop(**over) == ta.TA_ERR_INVALID_ARG


@host_only
def test_dropout_bwd_head_dims():
    assert call_bwd_drop(d=32) == ta.TA_ERR_UNSUPPORTED


@host_only
@pytest.mark.parametrize("field,off", [("do", 8), ("dk", 4), ("ws", 8), ("lse", 2)])
def test_dropout_bwd_misaligned(field, off):
    assert call_bwd_drop(**{field: A + off}) == ta.TA_ERR_MISALIGNED


def call_bwd_ex(**over):
    args = dict({p: A for p in BWD_PTRS}, B=1, H=2, Nq=100, Nk=300, d=128, dvw=64, off=200,
                scale=0.09, causal=1)
    args.update(over)
    return ta.attn_bwd_ex_raw(*(args[p] for p in BWD_PTRS), args["B"], args["H"], args["Nq"],
                              args["Nk"], args["d"], args["dvw"], args["off"], args["scale"],
                              args["causal"], 0)


@host_only
@pytest.mark.parametrize("over", [dict(Nq=-1), dict(Nk=(1 << 22) + 1), dict(off=-1),
                                  dict(off=(1 << 30) + 1), dict(causal=3), dict(scale=math.nan),
                                  dict(B=0), dict(q=0), dict(k=0), dict(ws=0), dict(dk=0)])
def test_bwd_ex_invalid(over):
    assert call_bwd_ex(**over) == ta.TA_ERR_INVALID_ARG


@host_only
@pytest.mark.parametrize("over", [dict(d=32), dict(dvw=96)])
def test_bwd_ex_head_dims(over):
    assert call_bwd_ex(**over) == ta.TA_ERR_UNSUPPORTED


@host_only
@pytest.mark.parametrize("field,off", [("q", 8), ("v", 4), ("dv", 8), ("lse", 2), ("ws", 4)])
def test_bwd_ex_misaligned(field, off):
    assert call_bwd_ex(**{field: A + off}) == ta.TA_ERR_MISALIGNED


@host_only
def test_bwd_ex_empty_is_a_no_op():
    assert call_bwd_ex(Nq=0, Nk=0, **{p: 0 for p in BWD_PTRS}) == ta.TA_OK


@host_only
def test_bwd_square_entry_still_rejects_empty():
    lib = ta.load_library()
    assert ta.attn_bwd_raw(*([A] * 10), 1, 2, 0, 128, 0.1, 1, 0) == ta.TA_ERR_INVALID_ARG
    assert lib.attn_bwd_workspace_size(1, 2, 0) == 0


# ---- split-key forward ----------------------------------------------------------

def test_split_plan_sizes():
    ws = ta.attn_fwd_split_workspace_size
    assert ws(2, 8, 16, 32768, 128) > 0              # 16 workgroups: split
    assert ws(16, 32, 1, 8192, 128) > 0              # 512 workgroups, one query: split in two
    assert ws(2, 32, 1024, 8192, 128) == 0           # 512 workgroups, Nq > Nk/64: partials too big
    assert ws(2, 32, 128, 8192, 128) > 0             # 512 workgroups, Nq = Nk/64: split in two
    assert ws(2, 32, 8192, 8192, 128) == 0           # 4096 workgroups: no split
    assert ws(1, 1, 1, 300, 128) == 0                # fewer than 8 key tiles
    assert ws(1, 1, 0, 4096, 128) == 0               # no queries
    assert ws(0, 1, 1, 4096, 128) == 0 and ws(1, 1, 1, 4096, 96) == 0   # out of range
    # partial O (dv floats) and LSE per (split, row), each part 256-byte aligned
    n = ws(2, 8, 16, 32768, 64)
    assert n % 256 == 0 and n >= 2 * 8 * 16 * 65 * 4


SPLIT_PTRS = ["q", "k", "v", "o", "lse"]


def call_split(ws=A, ws_bytes=1 << 30, **over):
    args = dict({p: A for p in SPLIT_PTRS}, B=2, H=8, Nq=16, Nk=32768, d=128, dvw=128, off=32752,
                scale=0.09, causal=1)
    args.update(over)
    return ta.attn_fwd_split_raw(*(args[p] for p in SPLIT_PTRS), args["B"], args["H"], args["Nq"],
                                 args["Nk"], args["d"], args["dvw"], args["off"], args["scale"],
                                 args["causal"], ws, ws_bytes, 0)


@host_only
def test_split_workspace_checks():
    need = ta.attn_fwd_split_workspace_size(2, 8, 16, 32768, 128)
    assert call_split(ws=0) == ta.TA_ERR_INVALID_ARG
    assert call_split(ws_bytes=need - 1) == ta.TA_ERR_INVALID_ARG
    assert call_split(ws=A + 128) == ta.TA_ERR_MISALIGNED


@host_only
@pytest.mark.parametrize("over", [dict(Nq=-1), dict(off=-5), dict(causal=2), dict(q=0),
                                  dict(scale=math.inf)])
def test_split_invalid(over):
    assert call_split(**over) == ta.TA_ERR_INVALID_ARG


@host_only
def test_split_head_dims_and_alignment():
    assert call_split(d=32) == ta.TA_ERR_UNSUPPORTED
    assert call_split(o=A + 8) == ta.TA_ERR_MISALIGNED


# ---- the backward without a workspace (library scratch) ----------------------------

def noalloc(**over):
    args = dict(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A, B=1, H=2, N=128, d=128,
                scale=0.1, causal=1)
    args.update(over)
    return ta.attn_bwd_noalloc_raw(*(args[n] for n in ("q", "k", "v", "o", "lse", "do", "dq",
                                                       "dk", "dv", "B", "H", "N", "d", "scale",
                                                       "causal")), 0)


@host_only
def test_noalloc_rejects_sizes_beyond_its_scratch():
    """16 MiB of scratch holds 8 bytes per row of B*H*(N rounded up to a multiple of 4): 2^21 rows."""
    assert noalloc(B=1, H=1, N=(1 << 21) + 2) == ta.TA_ERR_TOO_LARGE
    assert noalloc(B=2, H=16, N=65538) == ta.TA_ERR_TOO_LARGE
    assert noalloc(B=64, H=1, N=32769) == ta.TA_ERR_TOO_LARGE      # rounded up to 32772 rows


@host_only
@pytest.mark.parametrize("over,status", [
    (dict(q=0), ta.TA_ERR_INVALID_ARG), (dict(dv=0), ta.TA_ERR_INVALID_ARG),
    (dict(N=0), ta.TA_ERR_INVALID_ARG), (dict(causal=2), ta.TA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), ta.TA_ERR_INVALID_ARG), (dict(d=96), ta.TA_ERR_UNSUPPORTED),
    (dict(dq=A + 8), ta.TA_ERR_MISALIGNED), (dict(lse=A + 2), ta.TA_ERR_MISALIGNED)])
def test_noalloc_argument_errors_before_any_hip_call(over, status):
    assert noalloc(**over) == status


# ---- general-shape dropout and FP8 entry points ----------------------------------

@host_only
def test_general_dropout_and_fp8_argument_errors():
    lib = ta.load_library()
    sc = ctypes.c_float(0.1)
    # attn_fwd_dropout_ex: q k v o lse B H Nq Nk d dv off scale causal seed t stream
    assert lib.attn_fwd_dropout_ex(A, A, A, A, A, 1, 2, 16, 100, 64, 64, 84, sc, 1, 7, 256, 0) \
        == ta.TA_ERR_INVALID_ARG
    assert lib.attn_fwd_dropout_ex(A, A, A, A, A, 1, 2, 16, 100, 96, 64, 84, sc, 1, 7, 26, 0) \
        == ta.TA_ERR_UNSUPPORTED
    assert lib.attn_fwd_dropout_ex(A, A, A, A, A, 1, 2, 16, 100, 64, 64, -1, sc, 1, 7, 26, 0) \
        == ta.TA_ERR_INVALID_ARG
    # attn_bwd_dropout_ex: ... workspace B H Nq Nk d dv off scale causal seed t stream
    assert lib.attn_bwd_dropout_ex(*([A] * 10), 1, 2, 16, 100, 64, 64, 84, sc, 1, 7, -1, 0) \
        == ta.TA_ERR_INVALID_ARG
    assert lib.attn_bwd_dropout_ex(*([A] * 9), 0, 1, 2, 16, 100, 64, 64, 84, sc, 1, 7, 26, 0) \
        == ta.TA_ERR_INVALID_ARG
    # attn_fwd_fp8_ex: q8 k8 v o lse qd kd B H Nq Nk d dv off scale causal stream
    assert lib.attn_fwd_fp8_ex(*([A] * 7), 1, 2, 16, 100, 96, 64, 84, sc, 1, 0) \
        == ta.TA_ERR_UNSUPPORTED                                   # d = 96
    assert lib.attn_fwd_fp8_ex(*([A] * 7), 1, 2, 16, 100, 128, 96, 84, sc, 1, 0) \
        == ta.TA_ERR_UNSUPPORTED                                   # dv = 96
    assert lib.attn_fwd_fp8_ex(*([A] * 5), 0, A, 1, 2, 16, 100, 128, 64, 84, sc, 1, 0) \
        == ta.TA_ERR_INVALID_ARG                                   # no q descale
    assert lib.attn_fwd_fp8_ex(*([A] * 7), 1, 2, 16, 100, 128, 64, 84, sc, 3, 0) \
        == ta.TA_ERR_INVALID_ARG                                   # causal flag
    assert lib.attn_fwd_fp8_ex(A + 4, *([A] * 6), 1, 2, 16, 100, 128, 64, 84, sc, 1, 0) \
        == ta.TA_ERR_MISALIGNED
