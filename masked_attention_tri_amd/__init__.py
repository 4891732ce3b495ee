"""masked_attention_tri_amd: MI355X (gfx950) forward pass of masked, biased
triangle attention.

Python face of libtriattn (include/triattn.h).  ``triangle_attention``
follows the signature of cuEquivariance's ``triangle_attention`` API page
(q, k, v, bias, mask=None, scale=None, return_aux=False, *, kv_lengths=None)
and adds ``block_mask`` for the BlockMask list format of the
tensorplay.nn.attention page.  PyTorch only supplies device memory and
streams; the computation runs in the library's HIP kernels, and there is no
fallback path.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple, Union

import torch

from . import _native
from ._native import (  # noqa: F401
    TRIATTN_BF16,
    TRIATTN_ERR_HIP,
    TRIATTN_ERR_INVALID_ARG,
    TRIATTN_ERR_UNSUPPORTED,
    TRIATTN_F16,
    TRIATTN_F32,
    TRIATTN_MASK_BLOCK,
    TRIATTN_MASK_DENSE,
    TRIATTN_MASK_KV_LENGTHS,
    TRIATTN_MASK_NONE,
    TRIATTN_MOD_CAUSAL,
    TRIATTN_MOD_NONE,
    TRIATTN_KV_PACKED,
    TRIATTN_OK,
    TRIATTN_QKV_PACKED,
    TRIATTN_QKV_SEPARATE,
    TRIATTN_VARLEN_CAUSAL,
    TRIATTN_VARLEN_NO_MASK,
    TRIATTN_VARLEN_PADDING,
    LibraryNotBuilt,
    TriAttnMask,
    TriAttnShape,
    TriAttnVarlen,
    load_library,
    tri_attn_bwd,
    tri_attn_bwd_workspace_size,
    tri_attn_check,
    tri_attn_fwd,
    tri_attn_fwd_bias_dtype,
    tri_attn_mask_to_kv_lengths,
    tri_attn_status_str,
    tri_attn_varlen_check,
    tri_attn_varlen_fwd,
)

__all__ = ["triangle_attention", "triangle_attention_backward", "triangle_attention_autograd",
           "triangle_attention_varlen", "mask_to_kv_lengths", "tri_attn_varlen_fwd",
           "tri_attn_varlen_check",
           "BlockMask", "causal_mask", "tri_attn_fwd", "tri_attn_fwd_bias_dtype", "tri_attn_bwd",
           "tri_attn_bwd_workspace_size",
           "tri_attn_check",
           "tri_attn_status_str",
           "tri_attn_mask_to_kv_lengths", "load_library"]


def causal_mask(b, h, q_idx, kv_idx):
    """The causal mask_mod (q_idx >= kv_idx), in the (b, h, q_idx, kv_idx)
    callable form of the BlockMask page.  Passing this function (or the
    string "causal") as ``mask_mod`` selects the library's causal predicate;
    other callables cannot cross the C ABI and are rejected."""
    return q_idx >= kv_idx


class BlockMask:
    """Block-sparse key mask in the list format of the tensorplay.nn.attention
    page: (kv_num_blocks, kv_indices) plus the optional (full_kv_num_blocks,
    full_kv_indices) pair whose blocks skip mask_mod.

    Tensors have shape (..., ROWS) and (..., ROWS, MAX_BLOCKS); up to three
    leading dims broadcast against (B, N, H) like numpy (size 1 or the full
    size).  BLOCK_SIZE is an int or, as the page writes it, the tuple
    (KV_BLOCK_SIZE, Q_BLOCK_SIZE).  mask_mod is None, "causal" or
    ``causal_mask``.
    """

    def __init__(self, kv_num_blocks, kv_indices, full_kv_num_blocks=None,
                 full_kv_indices=None, BLOCK_SIZE: Union[int, Tuple[int, int]] = 128,
                 mask_mod=None, seq_lengths: Optional[Tuple[int, int]] = None):
        if kv_indices.dim() < 2:
            raise RuntimeError("BlockMask kv_indices must have at least 2 dimensions")
        if (full_kv_num_blocks is None) != (full_kv_indices is None):
            raise AssertionError("full_kv_num_blocks and full_kv_indices must be given together")
        if isinstance(BLOCK_SIZE, int):
            kvb = qb = int(BLOCK_SIZE)
        else:
            kvb, qb = (int(x) for x in BLOCK_SIZE)
        if mask_mod is None or mask_mod == "none":
            mod = TRIATTN_MOD_NONE
        elif mask_mod == "causal" or mask_mod is causal_mask:
            mod = TRIATTN_MOD_CAUSAL
        else:
            raise ValueError("mask_mod must be None, 'causal' or masked_attention_tri_amd."
                             "causal_mask; arbitrary callables cannot cross the C ABI")
        self.kv_num_blocks = kv_num_blocks
        self.kv_indices = kv_indices
        self.full_kv_num_blocks = full_kv_num_blocks
        self.full_kv_indices = full_kv_indices
        self.kv_block = kvb
        self.q_block = qb
        self.mask_mod = mod
        self.seq_lengths = seq_lengths

    @classmethod
    def from_kv_blocks(cls, kv_num_blocks, kv_indices, full_kv_num_blocks=None,
                       full_kv_indices=None, BLOCK_SIZE: Union[int, Tuple[int, int]] = 128,
                       mask_mod=None, seq_lengths: Optional[Tuple[int, int]] = None):
        return cls(kv_num_blocks, kv_indices, full_kv_num_blocks, full_kv_indices, BLOCK_SIZE,
                   mask_mod, seq_lengths)

    @property
    def shape(self):
        """(*leading, Q_LEN, KV_LEN) of the dense mask this describes."""
        rows = self.kv_num_blocks.shape[-1]
        q_len, kv_len = self.seq_lengths or (rows * self.q_block,
                                              self.kv_indices.shape[-1] * self.kv_block)
        return (*self.kv_num_blocks.shape[:-1], q_len, kv_len)

    def numel(self) -> int:
        """Elements of the dense mask, not accounting for sparsity."""
        return math.prod(self.shape)

    def sparsity(self) -> float:
        """Percentage of blocks not computed (visited = union of both lists,
        duplicates and out-of-range ids ignored).  Metadata helper; reads the
        lists on their device with torch ops."""
        q_len, kv_len = self.shape[-2:]
        nkb = -(-kv_len // self.kv_block)
        rows = self.kv_num_blocks.shape[-1]
        visited = torch.zeros(*self.kv_num_blocks.shape, nkb + 1, dtype=torch.bool,
                              device=self.kv_num_blocks.device)
        pairs = [(self.kv_num_blocks, self.kv_indices)]
        if self.full_kv_num_blocks is not None:
            pairs.append((self.full_kv_num_blocks, self.full_kv_indices))
        for num, idx in pairs:
            j = torch.arange(idx.shape[-1], device=idx.device)
            live = j < num.unsqueeze(-1).clamp(min=0)
            ids = idx.long()
            ok = live & (ids >= 0) & (ids < nkb)
            tgt = torch.where(ok, ids, torch.full_like(ids, nkb))
            visited.scatter_(-1, tgt, torch.ones_like(tgt, dtype=torch.bool))
        total = visited[..., :nkb].numel()
        if total == 0:
            return 0.0
        return 100.0 * (1.0 - visited[..., :nkb].sum().item() / total)

    def _descriptor(self, B, N, H, Q, K, device):
        rows = -(-Q // self.q_block)
        tensors = [self.kv_num_blocks, self.kv_indices, self.full_kv_num_blocks,
                   self.full_kv_indices]
        if self.kv_num_blocks.shape[-1] != rows:
            raise ValueError(f"kv_num_blocks has {self.kv_num_blocks.shape[-1]} rows; "
                             f"Q={Q} with q block {self.q_block} needs {rows}")
        lead = tuple(self.kv_num_blocks.shape[:-1])
        if len(lead) > 3:
            raise ValueError("at most three leading (B, N, H) dims")
        lead = (1,) * (3 - len(lead)) + lead
        for size, full in zip(lead, (B, N, H)):
            if size not in (1, full):
                raise ValueError(f"leading dims {lead} do not broadcast against {(B, N, H)}")
        conv = []
        for t in tensors:
            if t is None:
                conv.append(None)
                continue
            if t.device != device:
                raise ValueError("block lists must be on the same device as q")
            t = t.to(torch.int32).contiguous()
            conv.append(t)
        # every list is read with the kv_num_blocks instance strides, so all
        # four must have the same leading shape (no separate broadcasting)
        if conv[2] is not None and tuple(conv[2].shape) != tuple(self.kv_num_blocks.shape):
            raise ValueError("full_kv_num_blocks must have kv_num_blocks' shape "
                             f"{tuple(self.kv_num_blocks.shape)}, got {tuple(conv[2].shape)}")
        for idx_t in (conv[1], conv[3]):
            if idx_t is not None and tuple(idx_t.shape[:-1]) != tuple(self.kv_num_blocks.shape):
                raise ValueError("index tensors must be (..., ROWS, MAX_BLOCKS)")
        lb, ln, lh = lead
        d = TriAttnMask()
        d.kind = TRIATTN_MASK_BLOCK
        d.mask_mod = self.mask_mod
        d.kv_num_blocks = conv[0].data_ptr()
        d.kv_indices = conv[1].data_ptr()
        d.full_kv_num_blocks = conv[2].data_ptr() if conv[2] is not None else None
        d.full_kv_indices = conv[3].data_ptr() if conv[3] is not None else None
        d.q_block = self.q_block
        d.kv_block = self.kv_block
        d.max_blocks = conv[1].shape[-1]
        d.full_max_blocks = conv[3].shape[-1] if conv[3] is not None else 1
        d.stride_h = 1 if lh == H and H > 1 else 0
        d.stride_n = lh if ln == N and N > 1 else 0
        d.stride_b = ln * lh if lb == B and B > 1 else 0
        return d, conv  # keep the converted tensors alive for the call


def _as5(x, name):
    if x is None:
        return None
    if x.dim() == 4:
        return x.unsqueeze(0)
    if x.dim() != 5:
        raise ValueError(f"{name} must be 4-D (B=1) or 5-D, got {tuple(x.shape)}")
    return x


def _dense16(t):
    """t contiguous and 16-byte aligned (the library's requirement for the
    tensors it reads in 16-byte pieces): a view at an unaligned offset is
    copied into a fresh allocation."""
    t = t.contiguous()
    return t if t.data_ptr() % 16 == 0 else t.clone()


def _prepare(q, k, v, bias, mask, kv_lengths, block_mask, bias_in_input_dtype=False):
    """Shape and dtype checks, 5-D views, contiguous copies, and the mask
    descriptor (with the tensors it points at, which must stay alive).  The
    bias is cast to fp32, or to q's 16-bit dtype with bias_in_input_dtype."""
    if mask is not None and kv_lengths is not None:
        raise ValueError("pass either mask or kv_lengths, not both")
    if block_mask is not None and (mask is not None or kv_lengths is not None):
        raise ValueError("block_mask cannot be combined with mask or kv_lengths")
    four_d = q.dim() == 4
    q5, k5, v5 = _as5(q, "q"), _as5(k, "k"), _as5(v, "v")
    bias5, mask5, len5 = _as5(bias, "bias"), _as5(mask, "mask"), _as5(kv_lengths, "kv_lengths")
    if q5.dtype not in _native.DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q5.dtype}")
    if k5.dtype != q5.dtype or v5.dtype != q5.dtype:
        raise ValueError("q, k and v must share one dtype")
    if not q5.is_cuda:
        raise ValueError("inputs must be on a GPU device (there is no CPU path)")
    if k5.device != q5.device or v5.device != q5.device:
        raise ValueError("q, k and v must be on one device")
    B, N, H, Q, D = q5.shape
    K = k5.shape[3]
    if tuple(k5.shape) != (B, N, H, K, D) or tuple(v5.shape) != (B, N, H, K, D):
        raise ValueError(f"k and v must be (B,N,H,K,D) = {(B, N, H, K, D)}")
    dev = q5.device
    q5, k5, v5 = _dense16(q5), _dense16(k5), _dense16(v5)
    if bias5 is not None:
        if tuple(bias5.shape) != (B, 1, H, Q, K):
            raise ValueError(f"bias must be (B,1,H,Q,K) = {(B, 1, H, Q, K)}")
        bias_t = q5.dtype if bias_in_input_dtype else torch.float32
        bias5 = bias5.to(device=dev, dtype=bias_t).contiguous()

    desc = None
    keep = []
    if mask5 is not None:
        if tuple(mask5.shape) != (B, N, 1, 1, K):
            raise ValueError(f"mask must be (B,N,1,1,K) = {(B, N, 1, 1, K)}")
        m = mask5.to(device=dev, dtype=torch.bool).contiguous().view(torch.uint8)
        keep.append(m)
        desc = TriAttnMask()
        desc.kind = TRIATTN_MASK_DENSE
        desc.dense = m.data_ptr()
    elif len5 is not None:
        if tuple(len5.shape) != (B, N, 1, 1, 1):
            raise ValueError(f"kv_lengths must be (B,N,1,1,1) = {(B, N, 1, 1, 1)}")
        ln = len5.to(device=dev, dtype=torch.int32).contiguous()
        keep.append(ln)
        desc = TriAttnMask()
        desc.kind = TRIATTN_MASK_KV_LENGTHS
        desc.kv_lengths = ln.data_ptr()
    elif block_mask is not None:
        desc, conv = block_mask._descriptor(B, N, H, Q, K, dev)
        keep.extend(conv)

    return four_d, q5, k5, v5, bias5, desc, keep


def triangle_attention(q, k, v, bias=None, mask=None, scale: Optional[float] = None,
                       return_aux: bool = False, *, kv_lengths=None,
                       block_mask: Optional[BlockMask] = None, stream=None,
                       bias_in_input_dtype: bool = False):
    """Attention_q = sum_k softmax_k(s Q_q.K_k + B_qk if key k is valid else
    -1e9) V_k over (B, N, H, Q, D) tensors.

    q (B,N,H,Q,D); k, v (B,N,H,K,D); bias (B,1,H,Q,K) (cast to fp32) or None;
    mask (B,N,1,1,K) (cast to bool) | kv_lengths (B,N,1,1,1) int32 |
    block_mask: at most one.  4-D inputs are accepted when B = 1.  scale None
    means 1/sqrt(D).  Returns O (q's dtype), or (O, lse, max) with fp32 lse
    and max of shape (B,N,H,Q,1) when return_aux.  Runs on `stream` (torch's
    current stream by default) and does not synchronise.

    bias_in_input_dtype: cast the bias to q's dtype (bf16/fp16) instead of
    fp32, as the triangle_attention page's newest kernels do for speed; the
    result is that of the fp32 path on the rounded bias.
    """
    if bias_in_input_dtype and q.dtype == torch.float32:
        raise ValueError("bias_in_input_dtype needs bf16 or fp16 inputs")
    four_d, q5, k5, v5, bias5, desc, keep = _prepare(q, k, v, bias, mask, kv_lengths,
                                                     block_mask, bias_in_input_dtype)
    B, N, H, Q, D = q5.shape
    K = k5.shape[3]
    dev = q5.device
    out = torch.empty_like(q5)
    lse = torch.empty(B, N, H, Q, 1, device=dev, dtype=torch.float32)
    mx = torch.empty(B, N, H, Q, 1, device=dev, dtype=torch.float32)
    shape = TriAttnShape(B, N, H, Q, K, D)
    s = math.nan if scale is None else float(scale)
    dt = _native.DTYPE_CODES[q5.dtype]
    bias_dt = dt if bias_in_input_dtype and bias5 is not None else TRIATTN_F32
    st = tri_attn_fwd_bias_dtype(shape, dt, q5, k5, v5, bias5, bias_dt, desc, s, out, lse, mx,
                                 stream)
    if st != TRIATTN_OK:
        raise RuntimeError(f"tri_attn_fwd: {tri_attn_status_str(st)}")
    if four_d:
        out, lse, mx = out.squeeze(0), lse.squeeze(0), mx.squeeze(0)
    return (out, lse, mx) if return_aux else out


def mask_to_kv_lengths(mask):
    """Right-padded (B,N,1,1,K) bool mask -> (B,N,1,1,1) int32 lengths
    (4-D (N,1,1,K) -> (N,1,1,1)).  Raises ValueError if a row is not a
    prefix (a masked key followed by a valid one).  Synchronises once to read
    that check."""
    four_d = mask.dim() == 4
    m5 = _as5(mask, "mask")
    if not m5.is_cuda:
        raise ValueError("mask must be on a GPU device")
    B, N = m5.shape[:2]
    K = m5.shape[-1]
    if tuple(m5.shape) != (B, N, 1, 1, K):
        raise ValueError("mask must be (B,N,1,1,K)")
    m = m5.to(torch.bool).contiguous().view(torch.uint8)
    lens = torch.empty(B, N, 1, 1, 1, device=m.device, dtype=torch.int32)
    bad = torch.empty(1, device=m.device, dtype=torch.int32)
    st = tri_attn_mask_to_kv_lengths(m, B * N, K, lens, bad)
    if st != TRIATTN_OK:
        raise RuntimeError(f"tri_attn_mask_to_kv_lengths: {tri_attn_status_str(st)}")
    if int(bad.item()) != 0:
        raise ValueError(f"{int(bad.item())} mask rows are not right-padded prefixes; "
                         "pass the dense mask instead")
    return lens.squeeze(0) if four_d else lens


def triangle_attention_backward(q, k, v, bias, out, dout, lse, mx, mask=None,
                                scale: Optional[float] = None, *, kv_lengths=None,
                                block_mask: Optional[BlockMask] = None, stream=None):
    """Gradients of O = triangle_attention(q, k, v, bias, mask, scale, ...)
    for the incoming gradient dout: returns (dq, dk, dv, dbias), dq/dk/dv in
    q's dtype and dbias fp32 of shape (B,1,H,Q,K) (None when bias is None).
    out, lse and mx are the forward's (O, lse, max) for the same arguments
    (from return_aux=True).  Every step runs in the library's HIP kernels;
    the library's workspace (its per-row data, and with a bias
    the planes of dBias partial sums it asks for) is allocated here.
    """
    four_d, q5, k5, v5, bias5, desc, keep = _prepare(q, k, v, bias, mask, kv_lengths,
                                                     block_mask)
    B, N, H, Q, D = q5.shape
    K = k5.shape[3]
    o5, g5 = _dense16(_as5(out, "out")), _dense16(_as5(dout, "dout"))
    if any(t.device != q5.device for t in (o5, g5, lse, mx)):
        raise ValueError("out, dout, lse and max must be on q's device")
    if tuple(o5.shape) != (B, N, H, Q, D) or tuple(g5.shape) != (B, N, H, Q, D):
        raise ValueError(f"out and dout must be (B,N,H,Q,D) = {(B, N, H, Q, D)}")
    if o5.dtype != q5.dtype or g5.dtype != q5.dtype:
        raise ValueError("out and dout must have q's dtype")
    lse5 = _as5(lse, "lse").to(torch.float32).contiguous()
    mx5 = _as5(mx, "max").to(torch.float32).contiguous()
    if lse5.numel() != B * N * H * Q or mx5.numel() != B * N * H * Q:
        raise ValueError("lse and max must hold one value per (b, n, h, q) row")
    dq, dk, dv = torch.empty_like(q5), torch.empty_like(k5), torch.empty_like(v5)
    dbias = (torch.empty(B, 1, H, Q, K, device=q5.device, dtype=torch.float32)
             if bias5 is not None else None)
    s = math.nan if scale is None else float(scale)
    shape = TriAttnShape(B, N, H, Q, K, D)
    ws_bytes = tri_attn_bwd_workspace_size(shape, dbias is not None)
    ws = torch.empty((ws_bytes + 3) // 4, device=q5.device, dtype=torch.float32) if ws_bytes else None
    st = tri_attn_bwd(shape, _native.DTYPE_CODES[q5.dtype], q5, k5, v5,
                      bias5, desc, s, o5, g5, lse5, mx5, dq, dk, dv, dbias, stream, workspace=ws)
    if st != TRIATTN_OK:
        raise RuntimeError(f"tri_attn_bwd: {tri_attn_status_str(st)}")
    if four_d:
        dq, dk, dv = dq.squeeze(0), dk.squeeze(0), dv.squeeze(0)
        dbias = dbias.squeeze(0) if dbias is not None else None
    return dq, dk, dv, dbias


class _TriangleAttentionFn(torch.autograd.Function):
    """Forward through tri_attn_fwd, backward through tri_attn_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, bias, mask, scale, kv_lengths, block_mask, bias_in_input_dtype):
        out, lse, mx = triangle_attention(q, k, v, bias, mask, scale, return_aux=True,
                                          kv_lengths=kv_lengths, block_mask=block_mask,
                                          bias_in_input_dtype=bias_in_input_dtype)
        # the backward recomputes the softmax from the bias the forward used
        used_bias = bias.to(q.dtype) if bias is not None and bias_in_input_dtype else bias
        ctx.save_for_backward(q, k, v, used_bias, out, lse, mx)
        ctx.mask, ctx.scale, ctx.kv_lengths, ctx.block_mask = mask, scale, kv_lengths, block_mask
        ctx.bias_dtype = None if bias is None else bias.dtype
        ctx.mark_non_differentiable(lse, mx)
        return out, lse, mx

    @staticmethod
    def backward(ctx, dout, _dlse, _dmx):
        q, k, v, bias, out, lse, mx = ctx.saved_tensors
        dq, dk, dv, dbias = triangle_attention_backward(
            q, k, v, bias, out, dout.to(q.dtype).contiguous(), lse, mx, ctx.mask, ctx.scale,
            kv_lengths=ctx.kv_lengths, block_mask=ctx.block_mask)
        if dbias is not None:
            dbias = dbias.to(ctx.bias_dtype)
        return dq, dk, dv, dbias, None, None, None, None, None


def triangle_attention_autograd(q, k, v, bias=None, mask=None, scale: Optional[float] = None,
                                return_aux: bool = False, *, kv_lengths=None,
                                block_mask: Optional[BlockMask] = None,
                                bias_in_input_dtype: bool = False):
    """triangle_attention with gradients: O (or (O, lse, max)) recorded for
    torch.autograd, whose backward runs tri_attn_bwd.  Gradients flow to q,
    k, v and bias (its gradient is summed over n and cast to bias's dtype);
    lse and max are not differentiable."""
    out, lse, mx = _TriangleAttentionFn.apply(q, k, v, bias, mask, scale, kv_lengths, block_mask,
                                              bias_in_input_dtype)
    return (out, lse, mx) if return_aux else out


_VARLEN_LAYOUTS = {"separate": TRIATTN_QKV_SEPARATE, "qkv_packed": TRIATTN_QKV_PACKED,
                   "kv_packed": TRIATTN_KV_PACKED}
_VARLEN_MASKS = {"no_mask": TRIATTN_VARLEN_NO_MASK, "padding": TRIATTN_VARLEN_PADDING,
                 "causal": TRIATTN_VARLEN_CAUSAL}


def triangle_attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q: int,
                              max_seqlen_kv: int, *, layout: str = "separate",
                              mask_type: str = "padding", scale: Optional[float] = None,
                              return_aux: bool = False, stream=None):
    """Attention over packed variable-length sequences, in the layouts of
    Transformer Engine's fused_attn.h (NVTE_QKV_Layout, NVTE_Mask_Type,
    cu_seqlens / max_seqlen arguments): each query row attends to the keys
    of its own sequence only.

    layout "separate": q [Tq, H, D], k and v [Tkv, H, D];
    "qkv_packed": q is one tensor [T, 3, H, D] (k, v, cu_seqlens_kv None);
    "kv_packed": q [Tq, H, D] and k is one tensor [Tkv, 2, H, D] (v None).
    cu_seqlens_q / _kv: int32 [batch + 1] row offsets.  mask_type "no_mask"
    and "padding" (the same for packed rows) or "causal" (key j of query i,
    both counted within the sequence, only if j <= i).  Returns out
    [Tq, H, D], or (out, lse, max) with fp32 [Tq, H] aux; rows outside every
    sequence are left unwritten.  No bias; every step runs in the library.
    """
    if layout not in _VARLEN_LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(_VARLEN_LAYOUTS)}")
    if mask_type not in _VARLEN_MASKS:
        raise ValueError(f"mask_type must be one of {sorted(_VARLEN_MASKS)}")
    if not q.is_cuda:
        raise ValueError("inputs must be on a GPU device (there is no CPU path)")
    if q.dtype not in _native.DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    if layout == "qkv_packed":
        if q.dim() != 4 or q.shape[1] != 3:
            raise ValueError("qkv_packed: q must be [T, 3, H, D]")
        total_q, _, H, D = q.shape
        total_kv = total_q
        tensors = [_dense16(q)]
        kk = vv = None
        cu_kv = None
    else:
        if q.dim() != 3:
            raise ValueError("q must be [Tq, H, D]")
        total_q, H, D = q.shape
        if layout == "kv_packed":
            if k is None or k.dim() != 4 or tuple(k.shape[1:]) != (2, H, D):
                raise ValueError("kv_packed: k must be [Tkv, 2, H, D]")
            kk, vv = _dense16(k), None
        else:
            if k is None or v is None or k.dim() != 3 or tuple(k.shape[1:]) != (H, D) \
                    or k.shape != v.shape:
                raise ValueError("separate: k and v must be [Tkv, H, D]")
            kk, vv = _dense16(k), _dense16(v)
        total_kv = kk.shape[0]
        tensors = [_dense16(q)]
        if cu_seqlens_kv is None:
            raise ValueError("cu_seqlens_kv is required for this layout")
        cu_kv = cu_seqlens_kv.to(device=dev, dtype=torch.int32).contiguous()
    for t in (kk, vv):
        if t is not None and t.dtype != q.dtype:
            raise ValueError("q, k and v must share one dtype")
        if t is not None and t.device != dev:
            raise ValueError("q, k and v must be on one device")
    cu_q = cu_seqlens_q.to(device=dev, dtype=torch.int32).contiguous()
    if cu_q.dim() != 1 or (cu_kv is not None and cu_kv.shape != cu_q.shape):
        raise ValueError("cu_seqlens must be 1-D [batch + 1] and of equal length")
    batch = cu_q.numel() - 1
    qq = tensors[0]
    out = torch.empty(total_q, H, D, device=dev, dtype=q.dtype)
    lse = torch.empty(total_q, H, device=dev, dtype=torch.float32)
    mx = torch.empty(total_q, H, device=dev, dtype=torch.float32)
    d = TriAttnVarlen()
    d.layout = _VARLEN_LAYOUTS[layout]
    d.mask_type = _VARLEN_MASKS[mask_type]
    d.batch, d.heads, d.head_dim = max(batch, 0), H, D
    d.total_q, d.total_kv = total_q, total_kv
    d.cu_seqlens_q = cu_q.data_ptr()
    d.cu_seqlens_kv = cu_kv.data_ptr() if cu_kv is not None else None
    d.max_seqlen_q, d.max_seqlen_kv = int(max_seqlen_q), int(max_seqlen_kv)
    s = math.nan if scale is None else float(scale)
    st = tri_attn_varlen_fwd(d, _native.DTYPE_CODES[q.dtype], qq, kk, vv, s, out, lse, mx, stream)
    if st != TRIATTN_OK:
        raise RuntimeError(f"tri_attn_varlen_fwd: {tri_attn_status_str(st)}")
    return (out, lse, mx) if return_aux else out
