"""ctypes front end of the fp64 C oracle (``triattn_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  The arithmetic lives
in the C file; this module only converts arrays to contiguous fp64/int32/uint8
buffers, calls it, and reshapes the results.

Definition followed: cuEquivariance "cuequivariance_torch.triangle_attention"
API page, the defining equation (masked logits replaced by -1e9, post-scale
bias, softmax over keys), with the "kv_lengths" and "mask" parameter notes, and
the BlockMask format of the "tensorplay.nn.attention" API page (Basics and
Details items 1-2).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

MASK_NONE = 0
MASK_DENSE = 1
MASK_KV_LENGTHS = 2
MASK_BLOCK = 3
MOD_NONE = 0
MOD_CAUSAL = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "triattn_oracle.c")
_LIB = os.path.join(_HERE, "libtriattn_oracle.so")
_SRC_BWD = os.path.join(_HERE, "triattn_oracle_bwd.c")
_LIB_BWD = os.path.join(_HERE, "libtriattn_oracle_bwd.so")
_lib = None
_lib_bwd = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle with gcc (IEEE fp64, no fast-math)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-std=c11", "-Wall", "-Wextra",
           "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load_library(path: str):
    """Load a compiled oracle from ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    i64, ptr, c_int, dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.tri_oracle_fwd.restype = c_int
    lib.tri_oracle_fwd.argtypes = (
        [i64] * 6 + [ptr] * 4 + [c_int] + [ptr] * 6 + [i64] * 4 + [c_int] + [i64] * 3
        + [dbl, i64, ptr, ptr, ptr, ptr, c_int]
    )
    lib.tri_oracle_default_threads.restype = c_int
    lib.tri_oracle_default_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    _lib = load_library(_LIB)
    return _lib


def build_bwd(src: str = _SRC_BWD, out: str = _LIB_BWD) -> str:
    """Compile the backward oracle (its own library)."""
    return build(src, out)


def load_library_bwd(path: str):
    lib = ctypes.CDLL(path)
    i64, ptr, c_int, dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.tri_oracle_bwd.restype = c_int
    lib.tri_oracle_bwd.argtypes = (
        [i64] * 6 + [ptr] * 4 + [c_int] + [ptr] * 6 + [i64] * 4 + [c_int] + [i64] * 3
        + [dbl] + [ptr] * 5 + [i64, ptr, c_int]
    )
    return lib


def _load_bwd():
    global _lib_bwd
    if _lib_bwd is not None:
        return _lib_bwd
    if not os.path.exists(_LIB_BWD) or os.path.getmtime(_LIB_BWD) < os.path.getmtime(_SRC_BWD):
        build_bwd()
    _lib_bwd = load_library_bwd(_LIB_BWD)
    return _lib_bwd


def default_threads() -> int:
    return int(_load().tri_oracle_default_threads())


@dataclass
class OracleBlockMask:
    """Block-sparse key mask in the BlockMask list format.

    kv_num_blocks: (INST, ROWS) int; kv_indices: (INST, ROWS, MAX_BLOCKS) int;
    optional full_kv_* of the same leading shape.  ``instance`` strides map a
    (b, n, h) triple to a row of the leading INST axis; 0 broadcasts.
    """

    kv_num_blocks: np.ndarray
    kv_indices: np.ndarray
    full_kv_num_blocks: Optional[np.ndarray] = None
    full_kv_indices: Optional[np.ndarray] = None
    q_block: int = 128
    kv_block: int = 128
    mask_mod: int = MOD_NONE
    stride_b: int = 0
    stride_n: int = 0
    stride_h: int = 0


def _np(x, dtype):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: exact upcast on the CPU
        import torch

        x = x.detach().to("cpu")
        if dtype == np.float64:
            x = x.to(torch.float64)
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _mask_args(B, N, K, mask, kv_lengths, block):
    """Mask kind and the C arguments of one of the three mask forms."""
    given = sum(x is not None for x in (mask, kv_lengths, block))
    if given > 1:
        raise ValueError("pass at most one of mask, kv_lengths, block")

    kind = MASK_NONE
    dense = lens = None
    blk_args = [None] * 4 + [1, 1, 1, 1, MOD_NONE, 0, 0, 0]
    keep = []
    if mask is not None:
        m = _np(mask, np.uint8).reshape(B, N, K)
        dense = np.ascontiguousarray((m != 0).astype(np.uint8))
        kind = MASK_DENSE
    elif kv_lengths is not None:
        lens = _np(kv_lengths, np.int32).reshape(B, N)
        kind = MASK_KV_LENGTHS
    elif block is not None:
        kind = MASK_BLOCK
        nb = _np(block.kv_num_blocks, np.int32)
        ix = _np(block.kv_indices, np.int32)
        fnb = _np(block.full_kv_num_blocks, np.int32)
        fix = _np(block.full_kv_indices, np.int32)
        if (fnb is None) != (fix is None):
            raise ValueError("full_kv_num_blocks and full_kv_indices go together")
        keep += [nb, ix, fnb, fix]
        blk_args = [_ptr(nb), _ptr(ix), _ptr(fnb), _ptr(fix),
                    int(block.q_block), int(block.kv_block), int(ix.shape[-1]),
                    int(fix.shape[-1]) if fix is not None else 1,
                    int(block.mask_mod), int(block.stride_b), int(block.stride_n),
                    int(block.stride_h)]

    return kind, dense, lens, blk_args, keep


def oracle_fwd(q, k, v, bias=None, *, mask=None, kv_lengths=None,
               block: Optional[OracleBlockMask] = None, scale: Optional[float] = None,
               rows=None, threads: int = 0, lib=None):
    """Return (O, lse, max) in fp64.

    q: (B,N,H,Q,D); k, v: (B,N,H,K,D); bias: (B,1,H,Q,K) or None;
    mask: (B,N,K) or (B,N,1,1,K), nonzero = valid; kv_lengths: (B,N) or
    (B,N,1,1,1); block: OracleBlockMask.  At most one mask form may be given.
    rows: optional flat (b,n,h,q) row indices; then O is (len(rows), D) and
    lse/max are (len(rows),), else O is (B,N,H,Q,D) and lse/max (B,N,H,Q).
    ``lib`` selects another compiled copy of the oracle (used to check that
    the pins reject deliberately broken copies).
    """
    lib = lib or _load()
    qn, kn, vn = _np(q, np.float64), _np(k, np.float64), _np(v, np.float64)
    if qn.ndim != 5 or kn.ndim != 5 or vn.ndim != 5:
        raise ValueError("q, k, v must be 5-D (B,N,H,Q|K,D)")
    B, N, H, Q, D = qn.shape
    K = kn.shape[3]
    if kn.shape != (B, N, H, K, D) or vn.shape != kn.shape:
        raise ValueError("k/v shape mismatch")
    bn = _np(bias, np.float64)
    if bn is not None and bn.shape != (B, 1, H, Q, K):
        raise ValueError(f"bias must be (B,1,H,Q,K), got {bn.shape}")
    kind, dense, lens, blk_args, keep = _mask_args(B, N, K, mask, kv_lengths, block)

    if rows is None:
        n_rows = B * N * H * Q
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
        n_rows = rows_arr.size
    out = np.empty((n_rows, D), dtype=np.float64)
    lse = np.empty((n_rows,), dtype=np.float64)
    mx = np.empty((n_rows,), dtype=np.float64)
    s = math.nan if scale is None else float(scale)
    rc = lib.tri_oracle_fwd(B, N, H, Q, K, D, _ptr(qn), _ptr(kn), _ptr(vn), _ptr(bn),
                            kind, _ptr(dense), _ptr(lens), *blk_args, s, n_rows,
                            _ptr(rows_arr), _ptr(out), _ptr(lse), _ptr(mx), int(threads))
    if rc != 0:
        raise RuntimeError(f"tri_oracle_fwd failed with status {rc}")
    if rows is None:
        return out.reshape(B, N, H, Q, D), lse.reshape(B, N, H, Q), mx.reshape(B, N, H, Q)
    return out, lse, mx


def oracle_bwd(q, k, v, bias=None, *, dout, mask=None, kv_lengths=None,
               block: Optional[OracleBlockMask] = None, scale: Optional[float] = None,
               threads: int = 0, lib=None, q_rows=None):
    """Return (dQ, dK, dV, dBias) in fp64: the gradient of O = forward(q, k,
    v, bias) against the incoming gradient ``dout`` (B,N,H,Q,D).  dBias is
    (B,1,H,Q,K), or None without a bias.  Arguments as for oracle_fwd.

    q_rows: optional distinct query indices; only those rows of every
    (b,n,h) are evaluated, so dQ and dBias are exact on them (zero on the
    other rows) and dK, dV hold only their contributions."""
    lib = lib or _load_bwd()
    qn, kn, vn = _np(q, np.float64), _np(k, np.float64), _np(v, np.float64)
    B, N, H, Q, D = qn.shape
    K = kn.shape[3]
    if kn.shape != (B, N, H, K, D) or vn.shape != kn.shape:
        raise ValueError("k/v shape mismatch")
    bn = _np(bias, np.float64)
    if bn is not None and bn.shape != (B, 1, H, Q, K):
        raise ValueError(f"bias must be (B,1,H,Q,K), got {bn.shape}")
    gn = _np(dout, np.float64)
    if gn.shape != qn.shape:
        raise ValueError("dout must have q's shape")
    kind, dense, lens, blk_args, keep = _mask_args(B, N, K, mask, kv_lengths, block)
    dq = np.empty_like(qn)
    dk = np.empty_like(kn)
    dv = np.empty_like(vn)
    db = np.empty((B, 1, H, Q, K), dtype=np.float64) if bn is not None else None
    s = math.nan if scale is None else float(scale)
    qsel = None
    if q_rows is not None:
        qsel = np.ascontiguousarray(np.asarray(q_rows, dtype=np.int64).reshape(-1))
        if len(set(qsel.tolist())) != qsel.size:
            raise ValueError("q_rows must be distinct")
    rc = lib.tri_oracle_bwd(B, N, H, Q, K, D, _ptr(qn), _ptr(kn), _ptr(vn), _ptr(bn), kind,
                            _ptr(dense), _ptr(lens), *blk_args, s, _ptr(gn), _ptr(dq),
                            _ptr(dk), _ptr(dv), _ptr(db), 0 if qsel is None else qsel.size,
                            _ptr(qsel), int(threads))
    if rc != 0:
        raise RuntimeError(f"tri_oracle_bwd failed with status {rc}")
    return dq, dk, dv, db
