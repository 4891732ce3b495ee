"""ctypes view of libtriattn's C ABI (include/triattn.h).

Names mirror the C entry points.  This layer only converts torch tensors to
pointers and sizes; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing or cannot be
loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first, so the library shares it

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtriattn.so")

TRIATTN_OK = 0
TRIATTN_ERR_INVALID_ARG = 1
TRIATTN_ERR_UNSUPPORTED = 2
TRIATTN_ERR_HIP = 3

TRIATTN_F32 = 0
TRIATTN_F16 = 1
TRIATTN_BF16 = 2

TRIATTN_MASK_NONE = 0
TRIATTN_MASK_DENSE = 1
TRIATTN_MASK_KV_LENGTHS = 2
TRIATTN_MASK_BLOCK = 3

TRIATTN_MOD_NONE = 0
TRIATTN_MOD_CAUSAL = 1

EXPORTED = ("tri_attn_check", "tri_attn_fwd", "tri_attn_fwd_bias_dtype", "tri_attn_varlen_check",
            "tri_attn_varlen_fwd",
            "tri_attn_bwd", "tri_attn_bwd_workspace_size", "tri_attn_bwd_noalloc",
            "tri_attn_mask_to_kv_lengths", "tri_attn_status_str")

# bytes of the no-allocation backward's own workspace
TRIATTN_BWD_NOALLOC_BYTES = 48 * 1024 * 1024

TRIATTN_QKV_SEPARATE = 0
TRIATTN_QKV_PACKED = 1
TRIATTN_KV_PACKED = 2

TRIATTN_VARLEN_NO_MASK = 0
TRIATTN_VARLEN_PADDING = 1
TRIATTN_VARLEN_CAUSAL = 2

DTYPE_CODES = {torch.float32: TRIATTN_F32, torch.float16: TRIATTN_F16,
               torch.bfloat16: TRIATTN_BF16}


class TriAttnShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "N", "H", "Q", "K", "D")]


class TriAttnMask(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("mask_mod", ctypes.c_int32),
        ("dense", ctypes.c_void_p),
        ("kv_lengths", ctypes.c_void_p),
        ("kv_num_blocks", ctypes.c_void_p),
        ("kv_indices", ctypes.c_void_p),
        ("full_kv_num_blocks", ctypes.c_void_p),
        ("full_kv_indices", ctypes.c_void_p),
        ("q_block", ctypes.c_int64),
        ("kv_block", ctypes.c_int64),
        ("max_blocks", ctypes.c_int64),
        ("full_max_blocks", ctypes.c_int64),
        ("stride_b", ctypes.c_int64),
        ("stride_n", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
    ]


class TriAttnVarlen(ctypes.Structure):
    _fields_ = [
        ("layout", ctypes.c_int32),
        ("mask_type", ctypes.c_int32),
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("total_q", ctypes.c_int64),
        ("total_kv", ctypes.c_int64),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_kv", ctypes.c_void_p),
        ("max_seqlen_q", ctypes.c_int64),
        ("max_seqlen_kv", ctypes.c_int64),
    ]


_lib = None


class LibraryNotBuilt(RuntimeError):
    pass


def load_library(path: str = LIB_PATH):
    """Load libtriattn.so once; raise if it is absent (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LibraryNotBuilt(
            f"{path} is missing: build it with `python -m masked_attention_tri_amd.build` "
            "(there is no non-HIP implementation)")
    lib = ctypes.CDLL(path)
    P, I32, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    shape_p, mask_p = ctypes.POINTER(TriAttnShape), ctypes.POINTER(TriAttnMask)
    lib.tri_attn_check.restype = I32
    lib.tri_attn_check.argtypes = [shape_p, I32, P, P, P, P, mask_p, F32, P, P, P]
    lib.tri_attn_fwd.restype = I32
    lib.tri_attn_fwd.argtypes = [shape_p, I32, P, P, P, P, mask_p, F32, P, P, P, P]
    lib.tri_attn_fwd_bias_dtype.restype = I32
    lib.tri_attn_fwd_bias_dtype.argtypes = [shape_p, I32, P, P, P, P, I32, mask_p, F32, P, P, P, P]
    varlen_p = ctypes.POINTER(TriAttnVarlen)
    lib.tri_attn_varlen_check.restype = I32
    lib.tri_attn_varlen_check.argtypes = [varlen_p, I32, P, P, P, F32, P, P, P]
    lib.tri_attn_varlen_fwd.restype = I32
    lib.tri_attn_varlen_fwd.argtypes = [varlen_p, I32, P, P, P, F32, P, P, P, P]
    lib.tri_attn_bwd.restype = I32
    lib.tri_attn_bwd.argtypes = [shape_p, I32, P, P, P, P, mask_p, F32, P, P, P, P, P, P, P, P, P,
                                  ctypes.c_size_t, P]
    lib.tri_attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.tri_attn_bwd_workspace_size.argtypes = [shape_p, I32]
    lib.tri_attn_bwd_noalloc.restype = I32
    lib.tri_attn_bwd_noalloc.argtypes = [shape_p, I32, P, P, P, P, mask_p, F32, P, P, P, P, P, P,
                                         P, P, P]
    lib.tri_attn_mask_to_kv_lengths.restype = I32
    lib.tri_attn_mask_to_kv_lengths.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, P, P]
    lib.tri_attn_status_str.restype = ctypes.c_char_p
    lib.tri_attn_status_str.argtypes = [I32]
    _lib = lib
    return lib


def tri_attn_status_str(status: int) -> str:
    return load_library().tri_attn_status_str(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def tri_attn_check(shape: TriAttnShape, dtype: int, q, k, v, bias, mask, scale: float, out,
                   lse, mx) -> int:
    """Host-only validation (no device calls); returns the status code.

    q, k, v, bias, out, lse, mx are tensors or None; mask is a TriAttnMask or
    None.  Raw integer addresses may be passed instead of tensors.
    """
    conv = [ctypes.c_void_p(x) if isinstance(x, int) else _ptr(x)
            for x in (q, k, v, bias, out, lse, mx)]
    return int(load_library().tri_attn_check(
        ctypes.byref(shape), int(dtype), conv[0], conv[1], conv[2], conv[3],
        ctypes.byref(mask) if mask is not None else None, ctypes.c_float(scale),
        conv[4], conv[5], conv[6]))


def tri_attn_fwd(shape: TriAttnShape, dtype: int, q, k, v, bias, mask, scale: float, out, lse,
                 mx, stream) -> int:
    """Enqueue the forward pass on `stream` (a torch.cuda.Stream, a raw
    hipStream_t integer, or None for torch's current stream)."""
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return int(load_library().tri_attn_fwd(
        ctypes.byref(shape), int(dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
        ctypes.byref(mask) if mask is not None else None, ctypes.c_float(scale), _ptr(out),
        _ptr(lse), _ptr(mx), ctypes.c_void_p(handle)))


def tri_attn_fwd_bias_dtype(shape: TriAttnShape, dtype: int, q, k, v, bias, bias_dtype: int,
                            mask, scale: float, out, lse, mx, stream) -> int:
    """tri_attn_fwd with the bias of element type `bias_dtype` (TRIATTN_F32,
    or q's 16-bit type)."""
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return int(load_library().tri_attn_fwd_bias_dtype(
        ctypes.byref(shape), int(dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(bias), int(bias_dtype),
        ctypes.byref(mask) if mask is not None else None, ctypes.c_float(scale), _ptr(out),
        _ptr(lse), _ptr(mx), ctypes.c_void_p(handle)))


def _addr(x):
    return ctypes.c_void_p(x) if isinstance(x, int) else _ptr(x)


def tri_attn_varlen_check(desc: TriAttnVarlen, dtype: int, q, k, v, scale: float, out, lse,
                          mx) -> int:
    """Host-only validation of a packed-sequence forward (tensors, raw
    addresses or None)."""
    return int(load_library().tri_attn_varlen_check(
        ctypes.byref(desc), int(dtype), _addr(q), _addr(k), _addr(v), ctypes.c_float(scale),
        _addr(out), _addr(lse), _addr(mx)))


def tri_attn_varlen_fwd(desc: TriAttnVarlen, dtype: int, q, k, v, scale: float, out, lse, mx,
                        stream) -> int:
    """Enqueue the packed-sequence forward on `stream` (as tri_attn_fwd)."""
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return int(load_library().tri_attn_varlen_fwd(
        ctypes.byref(desc), int(dtype), _addr(q), _addr(k), _addr(v), ctypes.c_float(scale),
        _addr(out), _addr(lse), _addr(mx), ctypes.c_void_p(handle)))


def tri_attn_mask_to_kv_lengths(mask, rows: int, K: int, kv_lengths, nonprefix_rows,
                                stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(mask.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return int(load_library().tri_attn_mask_to_kv_lengths(
        _ptr(mask), int(rows), int(K), _ptr(kv_lengths), _ptr(nonprefix_rows),
        ctypes.c_void_p(handle)))


def tri_attn_bwd(shape: TriAttnShape, dtype: int, q, k, v, bias, mask, scale: float, out, dout,
                 lse, mx, dq, dk, dv, dbias, stream, workspace=None) -> int:
    """Enqueue the backward pass on `stream` (as tri_attn_fwd); `workspace`
    is a device tensor of at least tri_attn_bwd_workspace_size(shape, False) bytes, up to
    tri_attn_bwd_workspace_size(shape, dbias is not None) (None is passed as
    NULL, which the library refuses unless there is no query row)."""
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return int(load_library().tri_attn_bwd(
        ctypes.byref(shape), int(dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
        ctypes.byref(mask) if mask is not None else None, ctypes.c_float(scale), _ptr(out),
        _ptr(dout), _ptr(lse), _ptr(mx), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias),
        _ptr(workspace),
        ctypes.c_size_t(0 if workspace is None else workspace.numel() * workspace.element_size()),
        ctypes.c_void_p(handle)))


def tri_attn_bwd_workspace_size(shape: TriAttnShape, with_dbias: bool = True) -> int:
    """Bytes of workspace tri_attn_bwd uses at most for `shape` (the per-row
    data, plus the dBias split's partial sums when with_dbias)."""
    return int(load_library().tri_attn_bwd_workspace_size(ctypes.byref(shape), int(bool(with_dbias))))


def tri_attn_bwd_noalloc(shape: TriAttnShape, dtype: int, q, k, v, bias, mask, scale: float, out,
                         dout, lse, mx, dq, dk, dv, dbias, stream) -> int:
    """tri_attn_bwd with the library's own workspace: no workspace argument
    and no allocation (see include/triattn.h)."""
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return int(load_library().tri_attn_bwd_noalloc(
        ctypes.byref(shape), int(dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
        ctypes.byref(mask) if mask is not None else None, ctypes.c_float(scale), _ptr(out),
        _ptr(dout), _ptr(lse), _ptr(mx), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias),
        ctypes.c_void_p(handle)))
