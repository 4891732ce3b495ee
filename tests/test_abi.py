"""C-ABI tests that need no GPU: the library loads, exports every entry point
declared in include/*.h, and tri_attn_check (a pure host function) returns
the documented status for each invalid-argument case.  No compute call is
made here."""
import ctypes
import glob
import math
import os
import re

import pytest

import masked_attention_tri_amd as mat
from masked_attention_tri_amd import _native as nat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(tri_attn_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_entry_points():
    assert set(declared_functions()) == set(nat.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = mat.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), f"libtriattn.so does not export {name}"


def test_status_strings():
    for code in (0, 1, 2, 3):
        s = mat.tri_attn_status_str(code)
        assert s.startswith("TRIATTN_")
    assert "unknown" in mat.tri_attn_status_str(42)


A = 0x10000  # aligned fake addresses: tri_attn_check never dereferences them


def shape(B=1, N=2, H=2, Q=8, K=8, D=32):
    return nat.TriAttnShape(B, N, H, Q, K, D)


def check(shp=None, dtype=nat.TRIATTN_BF16, q=A, k=A, v=A, bias=A, mask=None, scale=math.nan,
          out=A, lse=A, mx=A):
    return nat.tri_attn_check(shp or shape(), dtype, q, k, v, bias, mask, scale, out, lse, mx)


def block_desc(**kw):
    d = nat.TriAttnMask()
    d.kind = nat.TRIATTN_MASK_BLOCK
    d.kv_num_blocks = A
    d.kv_indices = A
    d.q_block = d.kv_block = 128
    d.max_blocks = 4
    d.full_max_blocks = 4
    for key, val in kw.items():
        setattr(d, key, val)
    return d


def test_check_accepts_valid_arguments():
    assert check() == nat.TRIATTN_OK
    assert check(bias=0, lse=0, mx=0) == nat.TRIATTN_OK  # optional pointers
    assert check(shape(D=32), dtype=nat.TRIATTN_F32) == nat.TRIATTN_OK
    assert check(shape(D=128), dtype=nat.TRIATTN_F16) == nat.TRIATTN_OK
    assert check(shape(B=0, Q=0)) == nat.TRIATTN_OK  # empty work is fine
    assert check(mask=block_desc()) == nat.TRIATTN_OK
    assert check(mask=block_desc(full_kv_num_blocks=A, full_kv_indices=A)) == nat.TRIATTN_OK
    d = nat.TriAttnMask()
    d.kind = nat.TRIATTN_MASK_DENSE
    d.dense = A + 1  # byte mask: any alignment
    assert check(mask=d) == nat.TRIATTN_OK
    d = nat.TriAttnMask()
    d.kind = nat.TRIATTN_MASK_KV_LENGTHS
    d.kv_lengths = A
    assert check(mask=d) == nat.TRIATTN_OK


def test_check_empty_work_accepts_null_arrays():
    """No query row (B, N, H or Q is 0): the arrays an empty tensor hands over
    may be NULL; the other rules still apply."""
    none = dict(q=0, k=0, v=0, out=0, bias=0, lse=0, mx=0)
    for shp in (shape(N=0), shape(Q=0), shape(B=0), shape(H=0)):
        assert check(shp, **none) == nat.TRIATTN_OK
        for kind, field in ((nat.TRIATTN_MASK_DENSE, "dense"),
                            (nat.TRIATTN_MASK_KV_LENGTHS, "kv_lengths")):
            d = nat.TriAttnMask()
            d.kind = kind
            assert check(shp, mask=d, **none) == nat.TRIATTN_OK, field
        d = nat.TriAttnMask()
        d.kind = nat.TRIATTN_MASK_BLOCK
        d.q_block = d.kv_block = 128
        d.max_blocks = 4
        assert check(shp, mask=d, **none) == nat.TRIATTN_OK
        # still rejected: sizes, dtype, scale, both mask sources at once
        assert check(shape(N=0, K=0), **none) == nat.TRIATTN_ERR_INVALID_ARG
        assert check(shp, dtype=9, **none) == nat.TRIATTN_ERR_INVALID_ARG
        assert check(shp, scale=math.inf, **none) == nat.TRIATTN_ERR_INVALID_ARG
        d = nat.TriAttnMask()
        d.kind = nat.TRIATTN_MASK_DENSE
        d.kv_lengths = A
        assert check(shp, mask=d, **none) == nat.TRIATTN_ERR_INVALID_ARG
    # with a query row the NULL arrays are errors again
    assert check(q=0) == nat.TRIATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(v=0), dict(out=0),
    dict(q=A + 8), dict(out=A + 2), dict(bias=A + 2), dict(lse=A + 1), dict(mx=A + 3),
    dict(dtype=7), dict(dtype=-1),
    dict(shp=shape(K=0)), dict(shp=shape(D=0)), dict(shp=shape(B=-1)), dict(shp=shape(Q=-2)),
    dict(scale=math.inf), dict(scale=-math.inf),
])
def test_check_invalid_args(kw):
    assert check(**kw) == nat.TRIATTN_ERR_INVALID_ARG


def test_check_rejects_shape_null():
    lib = mat.load_library()
    assert lib.tri_attn_check(None, 2, A, A, A, A, None, 1.0, A, A, A) == \
        nat.TRIATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("dtype,D", [
    (nat.TRIATTN_F32, 36), (nat.TRIATTN_F32, 30), (nat.TRIATTN_F32, 64),
    (nat.TRIATTN_BF16, 264), (nat.TRIATTN_F16, 60), (nat.TRIATTN_BF16, 4),
    (nat.TRIATTN_F16, 260),
])
def test_check_envelope(dtype, D):
    # triangle_attention page, Notes item 3: fp32 D<=32, D%4==0; half types
    # D<=256 (the page's forward bound for its newest kernels), D%8==0
    assert check(shape(D=D), dtype=dtype) == nat.TRIATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype,D", [(nat.TRIATTN_BF16, 136), (nat.TRIATTN_F16, 256),
                                     (nat.TRIATTN_BF16, 8), (nat.TRIATTN_F32, 32)])
def test_check_envelope_accepts(dtype, D):
    assert check(shape(D=D), dtype=dtype) == nat.TRIATTN_OK


def test_check_mask_descriptors():
    both = nat.TriAttnMask()
    both.kind = nat.TRIATTN_MASK_DENSE
    both.dense = A
    both.kv_lengths = A  # a dense mask and kv_lengths together
    assert check(mask=both) == nat.TRIATTN_ERR_INVALID_ARG
    both.kind = nat.TRIATTN_MASK_KV_LENGTHS
    assert check(mask=both) == nat.TRIATTN_ERR_INVALID_ARG
    missing = nat.TriAttnMask()
    missing.kind = nat.TRIATTN_MASK_DENSE
    assert check(mask=missing) == nat.TRIATTN_ERR_INVALID_ARG
    missing.kind = nat.TRIATTN_MASK_KV_LENGTHS
    assert check(mask=missing) == nat.TRIATTN_ERR_INVALID_ARG
    bad_kind = nat.TriAttnMask()
    bad_kind.kind = 9
    assert check(mask=bad_kind) == nat.TRIATTN_ERR_INVALID_ARG
    lens = nat.TriAttnMask()
    lens.kind = nat.TRIATTN_MASK_KV_LENGTHS
    lens.kv_lengths = A + 2
    assert check(mask=lens) == nat.TRIATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(kv_num_blocks=None), dict(kv_indices=None),
    dict(full_kv_num_blocks=A),        # only one of the full pair
    dict(full_kv_indices=A),
    dict(max_blocks=0), dict(q_block=0), dict(kv_block=0),
    dict(full_kv_num_blocks=A, full_kv_indices=A, full_max_blocks=0),
    dict(mask_mod=5), dict(stride_b=-1), dict(stride_h=-3),
    dict(kv_indices=A + 2), dict(dense=A),
])
def test_check_block_descriptor(kw):
    assert check(mask=block_desc(**kw)) == nat.TRIATTN_ERR_INVALID_ARG


def test_check_block_count_limit():
    d = block_desc(kv_block=1)
    assert check(shape(K=8192), mask=d) == nat.TRIATTN_OK
    assert check(shape(K=8193), mask=d) == nat.TRIATTN_ERR_UNSUPPORTED


def test_check_index_range():
    assert check(shape(B=1 << 20, N=1 << 20, H=1 << 20, Q=2)) == nat.TRIATTN_ERR_UNSUPPORTED
    assert check(shape(B=1 << 62, N=4)) == nat.TRIATTN_ERR_UNSUPPORTED


def test_blockmask_constructor_errors():
    import torch

    with pytest.raises(RuntimeError):
        mat.BlockMask.from_kv_blocks(torch.zeros(4, dtype=torch.int32),
                                     torch.zeros(4, dtype=torch.int32))
    with pytest.raises(AssertionError):
        mat.BlockMask.from_kv_blocks(torch.zeros(4, dtype=torch.int32),
                                     torch.zeros(4, 2, dtype=torch.int32),
                                     full_kv_num_blocks=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError):
        mat.BlockMask.from_kv_blocks(torch.zeros(4, dtype=torch.int32),
                                     torch.zeros(4, 2, dtype=torch.int32),
                                     mask_mod=lambda b, h, q, k: q >= k)


def test_blockmask_rejects_mis_shaped_full_counts():
    """The kernels read every list with kv_num_blocks' instance strides, so a
    full_kv_num_blocks with other leading dims (e.g. broadcast (ROWS,) while
    kv_num_blocks is per (b, n, h)) is rejected on the host, before any
    launch."""
    import torch

    B, N, H, rows, width = 2, 3, 2, 4, 4
    num = torch.ones(B, N, H, rows, dtype=torch.int32)
    idx = torch.zeros(B, N, H, rows, width, dtype=torch.int32)
    good = mat.BlockMask.from_kv_blocks(num, idx, num.clone(), idx.clone(), BLOCK_SIZE=16)
    good._descriptor(B, N, H, 64, 64, torch.device("cpu"))
    bad = mat.BlockMask.from_kv_blocks(num, idx, torch.ones(rows, dtype=torch.int32),
                                       idx.clone(), BLOCK_SIZE=16)
    with pytest.raises(ValueError, match="full_kv_num_blocks"):
        bad._descriptor(B, N, H, 64, 64, torch.device("cpu"))
    bad_idx = mat.BlockMask.from_kv_blocks(num, idx, num.clone(),
                                           torch.zeros(rows, width, dtype=torch.int32),
                                           BLOCK_SIZE=16)
    with pytest.raises(ValueError):
        bad_idx._descriptor(B, N, H, 64, 64, torch.device("cpu"))


def test_blockmask_numel_and_sparsity():
    import torch

    rows = 4
    num = torch.arange(1, rows + 1, dtype=torch.int32)
    idx = torch.zeros(rows, rows, dtype=torch.int32)
    for i in range(rows):
        idx[i, : i + 1] = torch.arange(i + 1)
    bm = mat.BlockMask.from_kv_blocks(num, idx, BLOCK_SIZE=16, mask_mod="causal")
    assert bm.numel() == 64 * 64
    # causal lists visit 10 of 16 blocks
    assert abs(bm.sparsity() - 100.0 * 6 / 16) < 1e-9


def test_triangle_attention_argument_errors():
    import torch

    q = torch.zeros(1, 2, 2, 4, 8)
    with pytest.raises(ValueError):
        mat.triangle_attention(q, q, q, None, mask=torch.ones(1, 2, 1, 1, 4, dtype=torch.bool),
                               kv_lengths=torch.ones(1, 2, 1, 1, 1, dtype=torch.int32))
    with pytest.raises(ValueError):  # there is no CPU path
        mat.triangle_attention(q, q, q, None)


def _bwd(shp, dbias=A, ws=None, ws_bytes=0):
    lib = nat.load_library()
    return lib.tri_attn_bwd(ctypes.byref(shp), nat.TRIATTN_BF16, A, A, A, A, None,
                            ctypes.c_float(math.nan), A, A, A, A, A, A, A, dbias, ws,
                            ctypes.c_size_t(ws_bytes), None)


def test_bwd_workspace_validation():
    """The workspace must hold the per-row data (260 bytes per (b, n, h)
    slice and 32-row tile, rounded up to 16: tri_attn_bwd_workspace_size)
    and be 16-byte aligned, with or without a bias gradient; a failing check
    launches nothing (these calls make no device call)."""
    shp = shape(B=1, N=2, H=2, Q=8, K=8, D=32)
    need = 260 * 1 * 2 * 2 * 1
    assert nat.tri_attn_bwd_workspace_size(shp) == need
    assert _bwd(shp, ws=A, ws_bytes=need - 1) == nat.TRIATTN_ERR_INVALID_ARG
    assert _bwd(shp, dbias=None, ws=A, ws_bytes=need - 1) == nat.TRIATTN_ERR_INVALID_ARG
    assert _bwd(shp, ws=None, ws_bytes=need) == nat.TRIATTN_ERR_INVALID_ARG
    assert _bwd(shp, ws=A + 4, ws_bytes=need) == nat.TRIATTN_ERR_INVALID_ARG
    # no query row: nothing to do, whatever the workspace
    assert _bwd(shape(Q=0), ws=None, ws_bytes=0) == nat.TRIATTN_OK
    # int64 overflow of the workspace size
    big = shape(B=1 << 20, N=1 << 20, H=1 << 12, Q=1 << 12, K=8, D=32)
    assert _bwd(big, ws=A, ws_bytes=0) == nat.TRIATTN_ERR_UNSUPPORTED
    assert nat.tri_attn_bwd_workspace_size(big) == 0
    assert nat.tri_attn_bwd_workspace_size(shape(B=-1)) == 0
    # with a bias gradient, whole B H Q K fp32 planes of partial sums on top
    head = shape(B=1, N=768, H=4, Q=768, K=768, D=64)
    rows = 260 * 768 * 4 * 24
    assert nat.tri_attn_bwd_workspace_size(head, False) == rows
    extra = nat.tri_attn_bwd_workspace_size(head, True) - rows
    assert extra > 0 and extra % (4 * 4 * 768 * 768) == 0


def _varlen(**kw):
    d = nat.TriAttnVarlen()
    d.layout, d.mask_type = kw.get("layout", 0), kw.get("mask_type", 1)
    d.batch, d.heads, d.head_dim = kw.get("batch", 2), kw.get("heads", 2), kw.get("D", 64)
    d.total_q, d.total_kv = kw.get("total_q", 10), kw.get("total_kv", 12)
    d.cu_seqlens_q = kw.get("cu_q", A)
    d.cu_seqlens_kv = kw.get("cu_kv", A)
    d.max_seqlen_q, d.max_seqlen_kv = kw.get("max_q", 8), kw.get("max_kv", 8)
    return d


def _vcheck(d, dtype=nat.TRIATTN_BF16, q=A, k=A, v=A, out=A, scale=math.nan):
    return nat.tri_attn_varlen_check(d, dtype, q, k, v, scale, out, None, None)


def test_varlen_check_accepts_every_layout():
    assert _vcheck(_varlen()) == nat.TRIATTN_OK
    assert _vcheck(_varlen(layout=nat.TRIATTN_QKV_PACKED, total_kv=10, cu_kv=None),
                   k=None, v=None) == nat.TRIATTN_OK
    assert _vcheck(_varlen(layout=nat.TRIATTN_KV_PACKED), v=None) == nat.TRIATTN_OK
    assert _vcheck(_varlen(mask_type=nat.TRIATTN_VARLEN_CAUSAL), dtype=nat.TRIATTN_F32,
                   ) == nat.TRIATTN_ERR_UNSUPPORTED  # D = 64 is past the fp32 envelope
    assert _vcheck(_varlen(D=32), dtype=nat.TRIATTN_F32) == nat.TRIATTN_OK
    # no work: pointers may be NULL
    for kw in ({"batch": 0}, {"heads": 0}, {"total_q": 0}, {"max_q": 0}):
        assert _vcheck(_varlen(cu_q=None, cu_kv=None, **kw), q=None, k=None, v=None,
                       out=None) == nat.TRIATTN_OK


@pytest.mark.parametrize("kw,ptrs", [
    ({"layout": 3}, {}), ({"mask_type": 7}, {}), ({"batch": -1}, {}), ({"D": 0}, {}),
    ({"max_kv": -1}, {}), ({"total_kv": -2}, {}), ({"cu_q": None}, {}), ({"cu_kv": None}, {}),
    ({}, {"q": None}), ({}, {"k": None}), ({}, {"v": None}), ({}, {"out": None}),
    ({}, {"q": A + 8}), ({"cu_q": A + 2}, {}),
    ({"layout": 2}, {"k": None}),
    ({"layout": 1, "total_kv": 11, "cu_kv": None}, {}),   # packed qkv: one row count
    ({"layout": 1, "total_kv": 10, "cu_kv": A + 64}, {}),  # packed qkv: one offset array
    ({}, {"scale": math.inf}),
])
def test_varlen_check_invalid_args(kw, ptrs):
    assert _vcheck(_varlen(**kw), **ptrs) == nat.TRIATTN_ERR_INVALID_ARG


def test_varlen_check_envelope_and_range():
    assert _vcheck(_varlen(D=68)) == nat.TRIATTN_ERR_UNSUPPORTED
    assert _vcheck(_varlen(D=264)) == nat.TRIATTN_ERR_UNSUPPORTED
    assert _vcheck(_varlen(total_q=1 << 31)) == nat.TRIATTN_ERR_UNSUPPORTED  # int32 offsets
    assert _vcheck(_varlen(batch=1 << 20, heads=1 << 12, max_q=1 << 12)) == \
        nat.TRIATTN_ERR_UNSUPPORTED


def test_fwd_bias_dtype_validation():
    """The bias may be fp32 or the inputs' own 16-bit type, nothing else;
    a failing check launches nothing (no device call here)."""
    lib = nat.load_library()
    shp = shape(D=64)

    def call(dtype, bias_dtype, bias=A):
        return lib.tri_attn_fwd_bias_dtype(ctypes.byref(shp), dtype, A, A, A, bias, bias_dtype,
                                           None, ctypes.c_float(math.inf), A, None, None, None)

    # an infinite scale makes every otherwise-valid call stop at the check,
    # so these return without touching the device
    assert call(nat.TRIATTN_BF16, nat.TRIATTN_BF16) == nat.TRIATTN_ERR_INVALID_ARG
    for dt, bdt in ((nat.TRIATTN_BF16, nat.TRIATTN_F16), (nat.TRIATTN_F16, nat.TRIATTN_BF16),
                    (nat.TRIATTN_F32, nat.TRIATTN_F32 + 7), (nat.TRIATTN_BF16, 9)):
        assert call(dt, bdt) == nat.TRIATTN_ERR_INVALID_ARG
    # fp32 inputs have no 16-bit bias
    assert lib.tri_attn_fwd_bias_dtype(ctypes.byref(shape(D=32)), nat.TRIATTN_F32, A, A, A, A,
                                       nat.TRIATTN_F16, None, ctypes.c_float(math.nan), A, None,
                                       None, None) == nat.TRIATTN_ERR_INVALID_ARG
    # a 16-bit bias must be 2-byte aligned (checked after the common checks)
    assert lib.tri_attn_fwd_bias_dtype(ctypes.byref(shape(B=0)), nat.TRIATTN_BF16, A, A, A, A + 1,
                                       nat.TRIATTN_BF16, None, ctypes.c_float(math.nan), A, None,
                                       None, None) == nat.TRIATTN_ERR_INVALID_ARG


def test_bwd_noalloc_rejects_problems_past_its_scratch():
    """The no-allocation backward holds the per-row data in its own
    TRIATTN_BWD_NOALLOC_BYTES: a larger problem is refused before any device
    call, with or without a bias gradient; argument errors come first."""
    lib = nat.load_library()

    def call(shp, dbias=A, scale=math.nan):
        return lib.tri_attn_bwd_noalloc(ctypes.byref(shp), nat.TRIATTN_BF16, A, A, A, A, None,
                                        ctypes.c_float(scale), A, A, A, A, A, A, A, dbias, None)

    big = shape(B=1, N=1025, H=8, Q=1024, K=8, D=64)
    assert nat.tri_attn_bwd_workspace_size(big, False) > nat.TRIATTN_BWD_NOALLOC_BYTES
    assert call(big) == nat.TRIATTN_ERR_UNSUPPORTED
    assert call(big, dbias=None) == nat.TRIATTN_ERR_UNSUPPORTED
    assert call(big, scale=math.inf) == nat.TRIATTN_ERR_INVALID_ARG
    fits = shape(B=1, N=768, H=4, Q=768, K=768, D=64)
    assert nat.tri_attn_bwd_workspace_size(fits, False) <= nat.TRIATTN_BWD_NOALLOC_BYTES
    assert call(shape(B=1, N=0, H=4, Q=256, K=129, D=64)) == nat.TRIATTN_OK  # no work