"""Seeded synthetic inputs for the triangle-attention forward.

This module only draws random tensors; it holds none of the attention
arithmetic, so both the GPU path and the CPU oracle can consume its output.

Recipe (one CPU ``torch.Generator`` per case, with the seed listed per workload):
  * draws in the fixed order q, k, v, bias, then the mask / kv_lengths;
  * q, k, v ~ N(0, 1) drawn in fp32, then rounded (RNE) to the case dtype;
  * bias ~ N(0, sigma^2) in fp32, shape (B, 1, H, Q, K), shared over N;
  * masks follow the shapes of the cuEquivariance triangle_attention page
    ("mask" (B,N,1,1,K) bool, "kv_lengths" (B,N,1,1,1) int32) and the
    BlockMask list format of the tensorplay.nn.attention page.

The five named workloads are the sizes the library is specified and measured
on; ``make_case`` builds smaller random cases of any shape for tests.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class BlockLists:
    """Block-sparse key mask in list form (BlockMask "kv" and "full_kv" pairs).

    Leading dims of every tensor are (B', N', H') with sizes B or 1, N or 1,
    H or 1 (size 1 broadcasts), followed by ROWS = ceil(Q / q_block) and, for
    the index tensors, MAX_BLOCKS.
    """

    kv_num_blocks: torch.Tensor
    kv_indices: torch.Tensor
    full_kv_num_blocks: Optional[torch.Tensor] = None
    full_kv_indices: Optional[torch.Tensor] = None
    q_block: int = 128
    kv_block: int = 128
    mask_mod: str = "none"  # "none" or "causal"


@dataclass
class Case:
    name: str
    dtype: torch.dtype
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    bias: Optional[torch.Tensor]
    mask: Optional[torch.Tensor] = None         # (B,N,1,1,K) bool
    kv_lengths: Optional[torch.Tensor] = None   # (B,N,1,1,1) int32
    block: Optional[BlockLists] = None
    scale: Optional[float] = None
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, N, H, Q, D = self.q.shape
        return B, N, H, Q, self.k.shape[3], D

    def to(self, device) -> "Case":
        def mv(x):
            return None if x is None else x.to(device)

        blk = None
        if self.block is not None:
            b = self.block
            blk = BlockLists(mv(b.kv_num_blocks), mv(b.kv_indices), mv(b.full_kv_num_blocks),
                             mv(b.full_kv_indices), b.q_block, b.kv_block, b.mask_mod)
        return Case(self.name, self.dtype, mv(self.q), mv(self.k), mv(self.v), mv(self.bias),
                    mv(self.mask), mv(self.kv_lengths), blk, self.scale, dict(self.meta))


def _qkv(gen, B, N, H, Q, K, D, dtype):
    q = torch.randn(B, N, H, Q, D, generator=gen).to(dtype)
    k = torch.randn(B, N, H, K, D, generator=gen).to(dtype)
    v = torch.randn(B, N, H, K, D, generator=gen).to(dtype)
    return q, k, v


def _bias(gen, B, H, Q, K, sigma):
    return torch.randn(B, 1, H, Q, K, generator=gen) * sigma


def causal_block_lists(gen, n_rows: int, q_block: int = 128, kv_block: int = 128,
                       tail: str = "random") -> BlockLists:
    """Causal BlockMask lists for Q = K = n_rows * block.

    Row i lists kv blocks 0..i (the diagonal block needs the elementwise
    causal mask_mod) and full blocks 0..i-1.  Entries past each count are
    filled with in-range but wrong block ids, so reading past the count would
    change the result.
    """
    width = n_rows
    kv_num = torch.arange(1, n_rows + 1, dtype=torch.int32)
    full_num = torch.arange(0, n_rows, dtype=torch.int32)
    kv_idx = torch.randint(0, n_rows, (n_rows, width), generator=gen, dtype=torch.int32)
    full_idx = torch.randint(0, n_rows, (n_rows, width), generator=gen, dtype=torch.int32)
    for i in range(n_rows):
        kv_idx[i, : i + 1] = torch.arange(0, i + 1, dtype=torch.int32)
        full_idx[i, :i] = torch.arange(0, i, dtype=torch.int32)
    return BlockLists(kv_num.view(1, 1, 1, n_rows), kv_idx.view(1, 1, 1, n_rows, width),
                      full_num.view(1, 1, 1, n_rows), full_idx.view(1, 1, 1, n_rows, width),
                      q_block, kv_block, "causal")


# key -> (description, seed, dtype, B, N, H, Q=K, D)
WORKLOADS = {
    "fp32_dense_ones": ("fp32 dense-ones B1 N32 H2 Q=K=32 D32", 1001, "f32", 1, 32, 2, 32, 32),
    "fp16_lens96": ("fp16 kv_lengths=96 B1 N128 H2 Q=K=128 D32", 1002, "f16", 1, 128, 2, 128,
                    32),
    "bf16_dense_half": ("bf16 dense Bernoulli(0.5) B1 N384 H4 Q=K=384 D32", 1003, "bf16", 1,
                        384, 4, 384, 32),
    "bf16_lens_d64": ("bf16 kv_lengths U{384..768 step 8} B1 N768 H4 Q=K=768 D64", 1004,
                      "bf16", 1, 768, 4, 768, 64),
    "bf16_causal_blocks_d128": ("bf16 causal BlockMask 128 no-bias B2 N1 H8 Q=K=4096 D128",
                                1005, "bf16", 2, 1, 8, 4096, 128),
    # not one of the five: the widest head dimension of the envelope, in the
    # headline's form
    "bf16_lens_d256": ("bf16 kv_lengths U{256..512 step 8} B1 N256 H4 Q=K=512 D256", 1006,
                       "bf16", 1, 256, 4, 512, 256),
}
HEADLINE = "bf16_lens_d64"


def make_workload(key: str) -> Case:
    """The five named workloads, bit-for-bit reproducible."""
    name, seed, dt, B, N, H, S, D = WORKLOADS[key]
    dtype = DTYPES[dt]
    gen = torch.Generator().manual_seed(seed)
    q, k, v = _qkv(gen, B, N, H, S, S, D, dtype)
    meta = {"workload": key}
    if key == "fp32_dense_ones":
        bias = _bias(gen, B, H, S, S, 1.0)
        mask = torch.ones(B, N, 1, 1, S, dtype=torch.bool)
        return Case(name, dtype, q, k, v, bias, mask=mask, scale=1.0 / 32 ** 0.5, meta=meta)
    if key == "fp16_lens96":
        bias = _bias(gen, B, H, S, S, 1.0)
        lens = torch.full((B, N, 1, 1, 1), 96, dtype=torch.int32)
        return Case(name, dtype, q, k, v, bias, kv_lengths=lens, scale=1.0 / 32 ** 0.5,
                    meta=meta)
    if key == "bf16_dense_half":
        bias = _bias(gen, B, H, S, S, 2.0)
        mask = torch.rand(B, N, 1, 1, S, generator=gen) < 0.5
        dead = torch.randperm(N, generator=gen)[:4]
        mask[:, dead] = False
        meta["fully_masked_rows"] = sorted(int(x) for x in dead)
        return Case(name, dtype, q, k, v, bias, mask=mask, meta=meta)
    if key == "bf16_lens_d64":
        bias = _bias(gen, B, H, S, S, 1.0)
        lens = (8 * torch.randint(48, 97, (B, N, 1, 1, 1), generator=gen)).to(torch.int32)
        return Case(name, dtype, q, k, v, bias, kv_lengths=lens, scale=1.0 / 8.0, meta=meta)
    if key == "bf16_lens_d256":
        bias = _bias(gen, B, H, S, S, 1.0)
        lens = (8 * torch.randint(32, 65, (B, N, 1, 1, 1), generator=gen)).to(torch.int32)
        return Case(name, dtype, q, k, v, bias, kv_lengths=lens, scale=1.0 / 16.0, meta=meta)
    if key == "bf16_causal_blocks_d128":
        block = causal_block_lists(gen, S // 128)
        return Case(name, dtype, q, k, v, None, block=block, scale=None, meta=meta)
    raise KeyError(key)


def make_case(B, N, H, Q, K, D, dtype="bf16", mask_kind="none", seed=0, bias=True,
              bias_sigma=1.0, scale=None, p_valid=0.5, len_range=None, q_block=None,
              kv_block=None, block_density=0.5, with_full=True, mask_mod="none",
              block_broadcast=False) -> Case:
    """A random case of any shape.

    mask_kind: "none" | "dense" | "kv_lengths" | "block".
    dense: Bernoulli(p_valid) keys; kv_lengths: uniform ints in len_range
    (default [-2, K+3], which exercises both clamps); block: random kv lists
    with the given density in shuffled order, sometimes with a duplicate and an
    out-of-range id inside the counted part, plus optional full lists drawn
    mostly from the listed blocks and sometimes from unlisted ones.
    """
    dtype_t = DTYPES[dtype] if isinstance(dtype, str) else dtype
    gen = torch.Generator().manual_seed(int(seed))
    q, k, v = _qkv(gen, B, N, H, Q, K, D, dtype_t)
    b = _bias(gen, B, H, Q, K, bias_sigma) if bias else None
    name = f"case B{B} N{N} H{H} Q{Q} K{K} D{D} {dtype} {mask_kind} seed{seed}"
    c = Case(name, dtype_t, q, k, v, b, scale=scale, meta={"seed": seed})
    if mask_kind == "dense":
        c.mask = torch.rand(B, N, 1, 1, K, generator=gen) < p_valid
    elif mask_kind == "kv_lengths":
        lo, hi = len_range if len_range is not None else (-2, K + 3)
        c.kv_lengths = torch.randint(lo, hi + 1, (B, N, 1, 1, 1), generator=gen).to(torch.int32)
    elif mask_kind == "block":
        qb = q_block or 16
        kb = kv_block or 16
        rows = -(-Q // qb)
        nkb = -(-K // kb)
        lead = (1, 1, 1) if block_broadcast else (B, N, H)
        width = nkb + 2  # room for duplicates / out-of-range ids
        listed = torch.rand(*lead, rows, nkb, generator=gen) < block_density
        kv_num = torch.zeros(*lead, rows, dtype=torch.int32)
        kv_idx = torch.randint(-1, nkb + 1, (*lead, rows, width), generator=gen,
                               dtype=torch.int32)
        full_num = torch.zeros(*lead, rows, dtype=torch.int32)
        full_idx = torch.randint(-1, nkb + 1, (*lead, rows, width), generator=gen,
                                 dtype=torch.int32)
        fullsel = torch.rand(*lead, rows, nkb, generator=gen) < 0.5
        # a few full blocks that the kv list does not name: the lists are
        # read as a union, so these are visited too
        extra = torch.rand(*lead, rows, nkb, generator=gen) < 0.15
        junk = torch.rand(*lead, rows, 2, generator=gen) < 0.5
        flat_l = listed.reshape(-1, nkb)
        flat_f = (fullsel & (listed | extra)).reshape(-1, nkb)
        flat_j = junk.reshape(-1, 2)
        kn, ki = kv_num.view(-1), kv_idx.view(-1, width)
        fn, fi = full_num.view(-1), full_idx.view(-1, width)
        for r in range(flat_l.shape[0]):
            ids = torch.nonzero(flat_l[r]).view(-1).to(torch.int32)
            ids = ids[torch.randperm(ids.numel(), generator=gen)]
            extra_ids = []
            if flat_j[r, 0] and ids.numel() > 0:
                extra_ids.append(int(ids[0]))        # a duplicate entry
            if flat_j[r, 1]:
                extra_ids.append(nkb if r % 2 else -1)  # an out-of-range id
            ids = torch.cat([ids, torch.tensor(extra_ids, dtype=torch.int32)])
            kn[r] = ids.numel()
            ki[r, : ids.numel()] = ids
            f = torch.nonzero(flat_f[r]).view(-1).to(torch.int32)
            fn[r] = f.numel()
            fi[r, : f.numel()] = f
        c.block = BlockLists(kv_num, kv_idx, full_num if with_full else None,
                             full_idx if with_full else None, qb, kb, mask_mod)
    elif mask_kind != "none":
        raise ValueError(mask_kind)
    return c
