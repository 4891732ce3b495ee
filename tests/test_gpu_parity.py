"""GPU parity: the HIP library against the fp64 oracle, element by element.

Every case is compared on every output row: small random shapes, and the
five named workloads at their full sizes (the launches the benchmark times).
"""
import math

import numpy as np
import pytest
import torch

import masked_attention_tri_amd as mat
from masked_attention_tri_amd import workloads as wl
from tests import helpers as hp
from tests.gpu_common import assert_parity, block_mask_of, errors, run_gpu, say

pytestmark = pytest.mark.gpu


# ---- the five named workloads -------------------------------------------

def test_fp32_dense_ones():
    say("fp32 dense-ones workload")
    assert_parity(wl.make_workload("fp32_dense_ones"))


def test_fp32_dense_ones_without_mask():
    say("fp32 workload without mask")
    c = wl.make_workload("fp32_dense_ones")
    c.mask = None
    assert_parity(c)


def test_fp16_lens96():
    say("fp16 kv_lengths=96 workload")
    assert_parity(wl.make_workload("fp16_lens96"))


def test_bf16_dense_half_with_fully_masked_rows():
    """Every row of the workload (B1 N384 H4 Q=K=384 D32) against the oracle."""
    say("bf16 dense-mask workload (all rows)")
    c = wl.make_workload("bf16_dense_half")
    gpu = run_gpu(c)
    assert_parity(c, gpu=gpu)
    # the fully masked rows: uniform weights over all K keys
    for n in c.meta["fully_masked_rows"]:
        assert torch.all(gpu[2][0, n] == -1.0e9)
        assert torch.all(gpu[1][0, n] == -1.0e9)


def test_bf16_lens_d64_headline_all_rows():
    """Every row of the headline workload (B1 N768 H4 Q=K=768 D64, 2.36 M
    query rows) against the oracle, from the launch the benchmark times."""
    say("bf16 kv_lengths N768 D64 workload (full size, all rows)")
    c = wl.make_workload("bf16_lens_d64")
    assert_parity(c, gpu=run_gpu(c))


def test_bf16_causal_blocks_d128_all_rows():
    """Every row of the block-sparse workload (B2 N1 H8 Q=K=4096 D128, causal
    BlockMask with full lists) against the oracle."""
    say("bf16 causal BlockMask Q4096 D128 workload (full size, all rows)")
    c = wl.make_workload("bf16_causal_blocks_d128")
    assert_parity(c, gpu=run_gpu(c))


def test_bf16_lens_d256_all_rows():
    """Every row of the D = 256 workload (B1 N256 H4 Q=K=512 D256, kv_lengths
    U{256..512 step 8}) against the oracle."""
    say("bf16 kv_lengths N256 D256 workload (full size, all rows)")
    c = wl.make_workload("bf16_lens_d256")
    assert_parity(c, gpu=run_gpu(c))


# ---- random shapes through both kernels ------------------------------------

MFMA_CASES = [
    # (B, N, H, Q, K, D, dtype, kind, extra)
    (2, 3, 2, 200, 150, 64, "bf16", "kv_lengths", {}),
    (1, 2, 3, 130, 200, 64, "f16", "dense", {}),
    (2, 2, 2, 129, 64, 32, "bf16", "none", {}),
    (1, 3, 2, 96, 77, 128, "bf16", "dense", {"bias_sigma": 2.0}),
    (1, 2, 2, 256, 256, 128, "f16", "kv_lengths", {"len_range": (0, 256)}),
    (2, 1, 2, 256, 320, 64, "bf16", "block", {"q_block": 128, "kv_block": 64,
                                               "mask_mod": "causal"}),
    (1, 2, 2, 256, 256, 32, "f16", "block", {"q_block": 128, "kv_block": 128}),
    (1, 2, 3, 384, 250, 64, "bf16", "block", {"q_block": 256, "kv_block": 64,
                                               "mask_mod": "causal", "block_broadcast": True}),
    # an odd number of query tiles per row (the tile order alternates ends)
    (2, 3, 2, 640, 640, 64, "bf16", "block", {"q_block": 128, "kv_block": 128,
                                               "mask_mod": "causal"}),
    (2, 2, 2, 100, 100, 64, "bf16", "none", {"bias": False, "scale": 0.3}),
    (1, 4, 2, 64, 1, 64, "bf16", "none", {}),
    (1, 2, 2, 1, 100, 128, "f16", "kv_lengths", {}),
    (1, 2, 2, 70, 33, 32, "bf16", "kv_lengths", {"len_range": (-3, 0)}),
    (1, 3, 2, 150, 130, 64, "bf16", "dense", {"p_valid": 0.02}),
    (1, 2, 2, 128, 131, 64, "bf16", "none", {}),  # K % 4 != 0: scalar bias loads
    # dense masks past 64 key tiles: the mask bits are rebuilt per 64 tiles
    (1, 1, 2, 64, 4200, 64, "bf16", "dense", {}),
    (1, 2, 1, 96, 2090, 32, "bf16", "dense", {"p_valid": 0.9}),
    # D = 256 (one wave per SIMD): several query tiles, ragged keys, every mask kind
    (1, 2, 2, 300, 333, 256, "bf16", "kv_lengths", {"len_range": (0, 333)}),
    (1, 2, 2, 130, 257, 256, "f16", "dense", {}),
    (1, 1, 2, 384, 384, 256, "bf16", "block", {"q_block": 128, "kv_block": 64,
                                                "mask_mod": "causal"}),
    (2, 1, 2, 64, 100, 256, "bf16", "none", {"bias": False, "scale": 0.3}),
]

# head dimensions between the MFMA widths (multiples of 8): the MFMA kernel
# at the next width of 32, 64, 128 or 256, the extra columns zero
PADDED_D_CASES = [
    (2, 2, 3, 37, 29, 8, "bf16", "kv_lengths", {}),
    (1, 2, 2, 50, 70, 24, "f16", "dense", {}),
    (1, 2, 2, 33, 41, 40, "bf16", "none", {}),
    (1, 2, 1, 20, 130, 120, "f16", "kv_lengths", {}),
    (1, 3, 2, 150, 200, 96, "bf16", "kv_lengths", {"len_range": (0, 200)}),
    (1, 2, 2, 130, 131, 72, "f16", "none", {}),  # K % 4 != 0: per-lane bias loads
    (1, 2, 2, 256, 320, 48, "bf16", "block", {"q_block": 128, "kv_block": 64,
                                               "mask_mod": "causal"}),
    (1, 2, 2, 100, 100, 200, "bf16", "dense", {"p_valid": 0.02}),  # rows with no valid key
    (1, 2, 2, 90, 90, 56, "bf16", "none", {"scale": 0.3}),
    (1, 2, 2, 40, 33, 192, "f16", "dense", {}),
]

# block masks at D = 128 (and a width padded to it): odd and single-tile
# visited counts, rows with no listed block, ragged Q and K, every bias
# form, an inexact scale
BLOCK_D128_CASES = [
    (1, 2, 2, 256, 300, 128, "bf16", "block", {"q_block": 128, "kv_block": 32,
                                                "block_density": 0.3}),
    (1, 2, 2, 200, 96, 128, "f16", "block", {"q_block": 128, "kv_block": 32,
                                              "block_density": 0.2, "with_full": False}),
    (1, 1, 2, 256, 256, 128, "bf16", "block", {"q_block": 128, "kv_block": 128,
                                                "bias": False, "mask_mod": "causal"}),
    (2, 1, 2, 384, 384, 128, "bf16", "block", {"q_block": 128, "kv_block": 64,
                                                "mask_mod": "causal", "scale": 0.3}),
    (1, 2, 2, 256, 200, 104, "bf16", "block", {"q_block": 128, "kv_block": 64,
                                                "mask_mod": "causal"}),
    (1, 2, 2, 130, 131, 128, "f16", "block", {"q_block": 128, "kv_block": 32}),  # scalar bias
]

# fp32 inputs on the fp32 MFMA kernel (no mask, lengths, dense masks, block
# masks of 32-, 64- or whole 128-row query blocks and 16-key or whole
# 32-key blocks):
# several 128-row query tiles and 32-key tiles with ragged tails, rows with no valid key (length 0, a 2%
# dense mask, sparse block lists), an inexact scale, no bias, widths below 32
FP32_MFMA_CASES = [
    (1, 2, 2, 256, 200, 32, "f32", "block", {"q_block": 128, "kv_block": 32, "mask_mod": "causal"}),
    (1, 2, 2, 300, 300, 16, "f32", "block", {"q_block": 128, "kv_block": 64, "block_density": 0.3}),
    (2, 1, 2, 256, 256, 8, "f32", "block", {"q_block": 256, "kv_block": 128, "mask_mod": "causal",
                                             "block_broadcast": True}),
    # 32- and 64-row query blocks (4 or 2 block rows per workgroup)
    (1, 2, 2, 200, 150, 32, "f32", "block", {"q_block": 64, "kv_block": 32, "mask_mod": "causal"}),
    (1, 2, 2, 130, 200, 16, "f32", "block", {"q_block": 32, "kv_block": 64, "block_density": 0.3}),
    (2, 1, 2, 96, 96, 8, "f32", "block", {"q_block": 32, "kv_block": 32, "mask_mod": "causal",
                                           "block_broadcast": True, "bias": False}),
    # 16-key blocks (two per key tile)
    (1, 2, 2, 150, 97, 32, "f32", "block", {"q_block": 128, "kv_block": 16, "mask_mod": "causal"}),
    (1, 2, 2, 100, 130, 16, "f32", "block", {"q_block": 64, "kv_block": 16, "block_density": 0.4}),
    (1, 2, 2, 300, 250, 28, "f32", "kv_lengths", {"len_range": (0, 250)}),
    (1, 3, 2, 150, 131, 32, "f32", "dense", {}),
    (1, 2, 2, 140, 70, 16, "f32", "dense", {"p_valid": 0.02}),
    (2, 2, 2, 129, 100, 8, "f32", "none", {"scale": 0.3}),
    (1, 2, 2, 200, 96, 32, "f32", "none", {"bias": False}),
    (2, 3, 2, 19, 23, 12, "f32", "dense", {}),
    (1, 2, 2, 40, 40, 32, "f32", "kv_lengths", {"len_range": (-2, 45)}),
    (1, 2, 2, 9, 1, 32, "f32", "none", {}),
]

# half types with 32- or 64-row query blocks or 16-key kv blocks on the MFMA
# kernel (2 or 4 block rows per 128-row workgroup, each with its own kv
# lists; two kv blocks per key tile): ragged Q
# (a last block row partly or wholly past Q), rows with no listed block,
# causal with full lists, broadcast lists, every width class, an inexact
# scale, no bias
MULTI_ROW_BLOCK_CASES = [
    (1, 2, 2, 200, 300, 64, "bf16", "block", {"q_block": 64, "kv_block": 32, "mask_mod": "causal"}),
    (1, 2, 2, 250, 260, 128, "f16", "block", {"q_block": 32, "kv_block": 64,
                                               "block_density": 0.3}),
    (2, 1, 2, 256, 256, 32, "bf16", "block", {"q_block": 32, "kv_block": 32, "mask_mod": "causal",
                                               "block_broadcast": True}),
    (1, 2, 2, 130, 100, 256, "bf16", "block", {"q_block": 64, "kv_block": 32,
                                                "block_density": 0.4, "with_full": False}),
    (1, 2, 2, 256, 200, 64, "bf16", "block", {"q_block": 32, "kv_block": 64, "mask_mod": "causal",
                                               "scale": 0.3}),
    (1, 2, 2, 100, 150, 40, "f16", "block", {"q_block": 64, "kv_block": 32, "mask_mod": "causal"}),
    (1, 1, 2, 160, 128, 64, "bf16", "block", {"q_block": 32, "kv_block": 32, "bias": False,
                                               "mask_mod": "causal"}),
    (1, 2, 2, 64, 64, 64, "bf16", "block", {"q_block": 32, "kv_block": 32}),
    # 16-key kv blocks (two per 32-key tile, each listed, full or causal on
    # its own), with every query block size of the variant
    (1, 2, 2, 200, 150, 64, "bf16", "block", {"q_block": 128, "kv_block": 16, "mask_mod": "causal"}),
    (1, 2, 2, 130, 97, 128, "f16", "block", {"q_block": 64, "kv_block": 16, "block_density": 0.4}),
    (2, 1, 2, 96, 120, 32, "bf16", "block", {"q_block": 32, "kv_block": 16, "mask_mod": "causal",
                                              "block_broadcast": True}),
    (1, 2, 2, 256, 64, 256, "bf16", "block", {"q_block": 256, "kv_block": 16, "mask_mod": "causal",
                                               "bias": False}),
]

# the generic kernel: block masks whose query blocks are not whole 128-row
# tiles or 32 / 64 rows, or whose kv blocks are neither 16 keys nor whole
# 32-key tiles
GENERIC_CASES = [
    (2, 2, 2, 40, 37, 16, "bf16", "block", {"q_block": 16, "kv_block": 8, "mask_mod": "causal"}),
    (1, 2, 2, 64, 64, 64, "bf16", "block", {"q_block": 96, "kv_block": 32}),
    (1, 1, 2, 30, 30, 4, "f32", "block", {"q_block": 8, "kv_block": 4, "mask_mod": "causal"}),
    # D = 256 (half types)
    (1, 2, 2, 70, 90, 256, "bf16", "kv_lengths", {}),
    (1, 2, 2, 30, 50, 256, "bf16", "dense", {"p_valid": 0.02}),
    (1, 1, 2, 64, 64, 136, "bf16", "block", {"q_block": 32, "kv_block": 16, "mask_mod": "causal"}),
]


def _case_id(c):
    B, N, H, Q, K, D, dt, kind, extra = c
    return f"B{B}N{N}H{H}Q{Q}K{K}D{D}-{dt}-{kind}" + ("-" + "-".join(
        f"{k}" for k in extra) if extra else "")


ALL_CASES = (MFMA_CASES + PADDED_D_CASES + BLOCK_D128_CASES + MULTI_ROW_BLOCK_CASES +
             FP32_MFMA_CASES + GENERIC_CASES)


@pytest.mark.parametrize("spec", ALL_CASES, ids=[_case_id(c) for c in ALL_CASES])
@pytest.mark.parametrize("seed", [1, 2])
def test_random_shapes(spec, seed):
    B, N, H, Q, K, D, dt, kind, extra = spec
    c = wl.make_case(B, N, H, Q, K, D, dt, kind, seed=seed, **extra)
    say(c.name)
    assert_parity(c)


def test_p1_example_shapes_and_lengths():
    """The triangle_attention page's example: fp16, seq 128, 2 heads, D 32,
    lengths 96 built as a right-padded mask and turned into kv_lengths."""
    import json
    import os

    import masked_attention_tri_amd as mat

    say("P1 example")
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "p1_example_shapes.json")))
    c = wl.make_workload("fp16_lens96")
    assert list(c.q.shape) == g["q_shape"] and list(c.bias.shape) == g["bias_shape"]
    pos = torch.arange(128)
    mask = (pos.view(1, 128) < 96).view(1, 128, 1, 1, 1) & (pos.view(1, 128) < 96).view(
        1, 1, 1, 1, 128)
    lens = mat.mask_to_kv_lengths(mask.cuda())
    assert list(lens.shape) == g["kv_lengths_shape"]
    expect = torch.where(pos < 96, 96, 0).view(1, 128, 1, 1, 1).to(torch.int32)
    assert torch.equal(lens.cpu(), expect)
    c.kv_lengths = lens.cpu()
    gpu = run_gpu(c)
    assert list(gpu[0].shape) == g["output_shape"]
    assert_parity(c, gpu=gpu)  # rows n >= 96 have no valid key


# ---- the bias in the inputs' 16-bit type ------------------------------------

HALF_BIAS_CASES = [
    (1, 3, 2, 200, 192, 64, "bf16", "kv_lengths", {}),
    (1, 2, 2, 130, 96, 32, "f16", "dense", {"bias_sigma": 2.0}),
    (1, 2, 2, 256, 256, 128, "bf16", "block", {"q_block": 128, "kv_block": 64,
                                                "mask_mod": "causal"}),
    (1, 2, 2, 100, 160, 256, "f16", "none", {"scale": 0.3}),
    (2, 2, 2, 100, 100, 64, "bf16", "none", {}),      # K % 8 != 0: the generic kernel
    (1, 2, 2, 70, 88, 40, "bf16", "kv_lengths", {}),  # D = 40 on the width-64 tiles
]


@pytest.mark.parametrize("spec", HALF_BIAS_CASES, ids=[_case_id(c) for c in HALF_BIAS_CASES])
def test_half_bias_matches_oracle_on_the_rounded_bias(spec):
    """bias_in_input_dtype: the result is that of the equation with the bias
    rounded to the input type (the oracle fed exactly those values), at the
    usual tolerances.  Against the fp32 bias the only extra error is that
    rounding, reported here (it is what the 16-bit mode trades)."""
    B, N, H, Q, K, D, dt, kind, extra = spec
    c = wl.make_case(B, N, H, Q, K, D, dt, kind, seed=17, **extra)
    say(f"half bias {c.name}")
    g = c.to("cuda")
    got = mat.triangle_attention(g.q, g.k, g.v, g.bias, mask=g.mask, scale=g.scale,
                                 return_aux=True, kv_lengths=g.kv_lengths,
                                 block_mask=block_mask_of(g), bias_in_input_dtype=True)
    torch.cuda.synchronize()
    got = tuple(x.cpu() for x in got)
    rounded = wl.Case(c.name + " (rounded bias)", c.dtype, c.q, c.k, c.v,
                      c.bias.to(c.dtype).float(), mask=c.mask, kv_lengths=c.kv_lengths,
                      block=c.block, scale=c.scale)
    assert_parity(rounded, gpu=got)
    # each 16-bit value is widened exactly, then the arithmetic is the fp32
    # path's: the same bits as the fp32 path given the rounded bias, when
    # both run on the same kernel (a 16-bit bias needs K % 8 == 0 for the
    # MFMA kernel's DMA, an fp32 one K % 4 == 0)
    if D not in (32, 64, 128, 256) or K % 8 == 0:
        ref = run_gpu(rounded)
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), "differs from the fp32 path"
    eo, el, em = errors(c, got)
    say(f"half bias {c.name}: against the fp32 bias err O {eo:.3g} lse {el:.3g} max {em:.3g}")


def test_fp32_bias_dtype_is_tri_attn_fwd():
    """tri_attn_fwd_bias_dtype with TRIATTN_F32 is tri_attn_fwd, bit for bit."""
    say("bias dtype fp32 == tri_attn_fwd")
    import masked_attention_tri_amd._native as nat

    c = wl.make_case(1, 2, 2, 96, 128, 64, "bf16", "kv_lengths", seed=3).to("cuda")
    B, N, H, Q, K, D = c.shape
    desc = nat.TriAttnMask()
    desc.kind = nat.TRIATTN_MASK_KV_LENGTHS
    desc.kv_lengths = c.kv_lengths.data_ptr()
    shp = nat.TriAttnShape(B, N, H, Q, K, D)
    res = []
    for typed in (False, True):
        out = torch.empty_like(c.q)
        lse = torch.empty(B, N, H, Q, device="cuda")
        mx = torch.empty(B, N, H, Q, device="cuda")
        if typed:
            st = mat.tri_attn_fwd_bias_dtype(shp, nat.TRIATTN_BF16, c.q, c.k, c.v, c.bias,
                                             nat.TRIATTN_F32, desc, math.nan, out, lse, mx, None)
        else:
            st = mat.tri_attn_fwd(shp, nat.TRIATTN_BF16, c.q, c.k, c.v, c.bias, desc, math.nan,
                                  out, lse, mx, None)
        torch.cuda.synchronize()
        assert st == mat.TRIATTN_OK
        res.append((out, lse, mx))
    assert all(torch.equal(a, b) for a, b in zip(*res))
