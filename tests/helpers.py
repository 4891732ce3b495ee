"""Test-side glue: run the oracle on a workloads.Case, build dense masks.

The per-element dense mask of a block-sparse case is rebuilt here from the
BlockMask lists with the reconstruction loop of the tensorplay.nn.attention
page (Basics: for every row, mark the first num_blocks_in_row[row] listed
blocks), then combined with mask_mod on blocks that are not listed as full
(Details item 2).  Ids outside the block range are skipped; that is the
reading adopted for ids the page leaves undefined.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as orc


def block_instance_strides(block, B, N, H):
    """Instance strides for lists with leading dims (B|1, N|1, H|1)."""
    lb, ln, lh = block.kv_num_blocks.shape[:3]
    sh = 1 if lh == H and H > 1 else 0
    sn = lh if ln == N and N > 1 else 0
    sb = ln * lh if lb == B and B > 1 else 0
    return sb, sn, sh


def oracle_block(case):
    b = case.block
    B, N, H, Q, K, D = case.shape
    sb, sn, sh = block_instance_strides(b, B, N, H)
    rows = b.kv_num_blocks.shape[3]
    return orc.OracleBlockMask(
        b.kv_num_blocks.reshape(-1, rows).cpu(),
        b.kv_indices.reshape(-1, rows, b.kv_indices.shape[-1]).cpu(),
        None if b.full_kv_num_blocks is None else b.full_kv_num_blocks.reshape(-1, rows).cpu(),
        None if b.full_kv_indices is None
        else b.full_kv_indices.reshape(-1, rows, b.full_kv_indices.shape[-1]).cpu(),
        q_block=b.q_block, kv_block=b.kv_block,
        mask_mod=orc.MOD_CAUSAL if b.mask_mod == "causal" else orc.MOD_NONE,
        stride_b=sb, stride_n=sn, stride_h=sh)


def run_oracle(case, rows=None, threads=0, scale="case", fwd=None):
    """Oracle (O, lse, max) in fp64 for a Case (inputs upcast exactly)."""
    fwd = fwd or orc.oracle_fwd
    s = case.scale if scale == "case" else scale
    kw = {}
    if case.mask is not None:
        kw["mask"] = case.mask
    elif case.kv_lengths is not None:
        kw["kv_lengths"] = case.kv_lengths
    elif case.block is not None:
        kw["block"] = oracle_block(case)
    return fwd(case.q, case.k, case.v, case.bias, scale=s, rows=rows, threads=threads, **kw)


def dense_from_blocks(case):
    """(B,N,H,Q,K) bool validity of a block-sparse case (reconstruction loop)."""
    b = case.block
    B, N, H, Q, K, D = case.shape
    nkb = -(-K // b.kv_block)
    rows = -(-Q // b.q_block)
    out = torch.zeros(B, N, H, Q, K, dtype=torch.bool)
    qi = torch.arange(Q).view(Q, 1)
    ki = torch.arange(K).view(1, K)
    for bb in range(B):
        for nn in range(N):
            for hh in range(H):
                ib = bb if b.kv_num_blocks.shape[0] > 1 else 0
                inn = nn if b.kv_num_blocks.shape[1] > 1 else 0
                ih = hh if b.kv_num_blocks.shape[2] > 1 else 0
                listed = torch.zeros(rows, nkb, dtype=torch.bool)
                full = torch.zeros(rows, nkb, dtype=torch.bool)
                pairs = [(b.kv_num_blocks, b.kv_indices, listed)]
                if b.full_kv_num_blocks is not None:
                    pairs.append((b.full_kv_num_blocks, b.full_kv_indices, full))
                for num_t, idx_t, dense_blocks in pairs:
                    num = num_t[ib, inn, ih]
                    idx = idx_t[ib, inn, ih]
                    for row in range(rows):
                        cnt = max(0, min(int(num[row]), idx.shape[-1]))
                        for j in range(cnt):
                            col = int(idx[row, j])
                            if 0 <= col < nkb:
                                dense_blocks[row, col] = True
                listed |= full
                blk_r = (torch.arange(Q) // b.q_block).view(Q, 1)
                blk_c = (torch.arange(K) // b.kv_block).view(1, K)
                lst = listed[blk_r, blk_c]
                ful = full[blk_r, blk_c]
                mod = (qi >= ki) if b.mask_mod == "causal" else torch.ones(Q, K, dtype=torch.bool)
                out[bb, nn, hh] = lst & (ful | mod)
    return out


def valid_matrix(case):
    """(B,N,H,Q,K) bool key validity for any mask kind."""
    B, N, H, Q, K, D = case.shape
    if case.mask is not None:
        m = case.mask.reshape(B, N, 1, 1, K).to(torch.bool)
        return m.expand(B, N, H, Q, K).clone()
    if case.kv_lengths is not None:
        lens = case.kv_lengths.reshape(B, N, 1, 1, 1).clamp(0, K)
        return (torch.arange(K).view(1, 1, 1, 1, K) < lens).expand(B, N, H, Q, K).clone()
    if case.block is not None:
        return dense_from_blocks(case)
    return torch.ones(B, N, H, Q, K, dtype=torch.bool)


def to_np(x):
    return x.detach().cpu().numpy() if hasattr(x, "detach") else np.asarray(x)
