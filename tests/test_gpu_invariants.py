"""GPU invariants of the library that hold at any size (mostly bitwise)."""
import math

import numpy as np
import pytest
import torch

import oracle as orc

import masked_attention_tri_amd as mat
from masked_attention_tri_amd import _native as nat
from masked_attention_tri_amd import workloads as wl
from tests.gpu_common import TOL, assert_parity, block_mask_of, run_gpu, say

pytestmark = pytest.mark.gpu


def _eq(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("D,dt", [(64, "bf16"), (32, "f16"), (24, "bf16"), (32, "f32")])
def test_default_scale_is_inv_sqrt_d(D, dt):
    say(f"default scale D={D} {dt}")
    c = wl.make_case(1, 2, 2, 70, 90, D, dt, "dense", seed=3)
    assert _eq(run_gpu(c, scale=None), run_gpu(c, scale=1.0 / math.sqrt(D)))


@pytest.mark.parametrize("D", [64, 40])
def test_kv_length_clamps(D):
    say(f"kv_lengths clamps D={D}")
    c = wl.make_case(1, 4, 2, 100, 90, D, "bf16", "kv_lengths", seed=4)
    c.kv_lengths = torch.tensor([90, 0, 17, 64], dtype=torch.int32).view(1, 4, 1, 1, 1)
    base = run_gpu(c)
    c2 = wl.Case(c.name, c.dtype, c.q, c.k, c.v, c.bias, scale=c.scale,
                 kv_lengths=torch.tensor([95, -3, 17, 64], dtype=torch.int32).view(1, 4, 1, 1, 1))
    assert _eq(base, run_gpu(c2))
    # a prefix dense mask gives the same answer
    dense = torch.arange(90).view(1, 1, 1, 1, 90) < c.kv_lengths
    c3 = wl.Case(c.name, c.dtype, c.q, c.k, c.v, c.bias, scale=c.scale, mask=dense)
    d = run_gpu(c3)
    tol = TOL[c.dtype]
    assert (d[0].float() - base[0].float()).abs().max() <= tol["o"]
    assert (d[1] - base[1]).abs().max() <= tol["lse"]


def test_full_lists_are_only_an_optimisation():
    say("full_kv lists on/off")
    g = torch.Generator().manual_seed(8)
    c = wl.make_case(2, 1, 2, 512, 512, 64, "bf16", "none", seed=8, bias=True)
    c.block = wl.causal_block_lists(g, 4, 128, 128)
    with_full = run_gpu(c)
    c.block = wl.BlockLists(c.block.kv_num_blocks, c.block.kv_indices, None, None, 128, 128,
                            "causal")
    without = run_gpu(c)
    assert _eq(with_full, without)
    assert_parity(c, gpu=without)


@pytest.mark.parametrize("key", ["fp16_lens96", "bf16_lens_d64"])
def test_run_to_run_determinism(key):
    say(f"determinism {key}")
    c = wl.make_workload(key)
    assert _eq(run_gpu(c), run_gpu(c))


@pytest.mark.parametrize("dt,D,kind,shape,extra", [
    ("bf16", 64, "kv_lengths", (2, 2, 2, 131, 77), {}),
    ("f16", 128, "dense", (2, 2, 2, 131, 77), {}),
    ("bf16", 24, "none", (2, 2, 2, 131, 77), {}),
    ("f32", 16, "dense", (2, 2, 2, 131, 77), {}),
    # many query tiles per row, ragged last tile, odd N
    ("bf16", 64, "kv_lengths", (1, 3, 2, 1000, 700), {"len_range": (0, 700)}),
    ("bf16", 32, "dense", (1, 5, 2, 1000, 300), {}),
    # block-sparse: 8 query tiles of a causal 128 x 64 BlockMask, and a
    # random one with duplicates and out-of-range ids
    ("bf16", 64, "block", (1, 2, 2, 1024, 1024),
     {"q_block": 128, "kv_block": 64, "mask_mod": "causal"}),
    ("f16", 128, "block", (2, 1, 2, 640, 600), {"q_block": 128, "kv_block": 128}),
    # sparse block lists (rows with none) at a padded width
    ("bf16", 120, "block", (1, 2, 2, 300, 250),
     {"q_block": 128, "kv_block": 32, "block_density": 0.15}),
    ("bf16", 256, "kv_lengths", (1, 3, 2, 300, 200), {"len_range": (0, 200)}),
    # 32-row query blocks (four block rows per workgroup), sparse lists
    ("bf16", 64, "block", (1, 2, 2, 300, 250),
     {"q_block": 32, "kv_block": 32, "block_density": 0.2}),
    # widths between the MFMA tiles: every one of the D columns is stored
    ("bf16", 96, "kv_lengths", (1, 3, 2, 300, 200), {"len_range": (0, 200)}),
    ("f16", 200, "dense", (1, 2, 2, 131, 77), {}),
])
def test_every_output_element_is_written(dt, D, kind, shape, extra):
    say(f"NaN-prefilled outputs {dt} D={D} {kind} {shape}")
    c = wl.make_case(*shape, D, dt, kind, seed=9, **extra).to("cuda")
    out = torch.full_like(c.q, float("nan"))
    lse = torch.full(c.q.shape[:4], float("nan"), device="cuda")
    mx = torch.full(c.q.shape[:4], float("nan"), device="cuda")
    desc = None
    if c.mask is not None:
        m = c.mask.contiguous().view(torch.uint8)
        desc = nat.TriAttnMask()
        desc.kind = nat.TRIATTN_MASK_DENSE
        desc.dense = m.data_ptr()
    elif c.kv_lengths is not None:
        ln = c.kv_lengths.contiguous()
        desc = nat.TriAttnMask()
        desc.kind = nat.TRIATTN_MASK_KV_LENGTHS
        desc.kv_lengths = ln.data_ptr()
    elif c.block is not None:
        desc, keep = block_mask_of(c)._descriptor(*c.shape[:5], c.q.device)
    B, N, H, Q, K, D = c.shape
    st = mat.tri_attn_fwd(nat.TriAttnShape(B, N, H, Q, K, D), nat.DTYPE_CODES[c.q.dtype],
                          c.q, c.k, c.v, c.bias, desc, math.nan, out, lse, mx, None)
    torch.cuda.synchronize()
    assert st == mat.TRIATTN_OK
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all() and \
        torch.isfinite(mx).all()


def test_optional_aux_outputs_and_invalid_args_write_nothing():
    say("null lse/max; rejected call writes nothing")
    c = wl.make_case(1, 2, 2, 64, 64, 64, "bf16", "none", seed=10).to("cuda")
    out = torch.zeros_like(c.q)
    B, N, H, Q, K, D = c.shape
    shp = nat.TriAttnShape(B, N, H, Q, K, D)
    assert mat.tri_attn_fwd(shp, nat.TRIATTN_BF16, c.q, c.k, c.v, c.bias, None, math.nan,
                            out, None, None, None) == mat.TRIATTN_OK
    torch.cuda.synchronize()
    ref = run_gpu(c.to("cpu"), scale=None)
    assert torch.equal(out.cpu(), ref[0])
    poison = torch.full_like(c.q, 7.0)
    bad = nat.TriAttnShape(B, N, H, Q, K, 68)  # D % 8 != 0: no 16-bit kernel takes it
    assert mat.tri_attn_fwd(bad, nat.TRIATTN_BF16, c.q, c.k, c.v, c.bias, None, math.nan,
                            poison, None, None, None) == mat.TRIATTN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(poison == 7.0)


def test_inputs_on_another_device_are_rejected():
    """Every tensor the binding hands to the library must live on q's
    device: a host tensor among them is an error, never a host pointer
    passed to a kernel."""
    say("inputs split across devices")
    c = wl.make_case(1, 2, 2, 32, 32, 32, "bf16", "kv_lengths", seed=12).to("cuda")
    with pytest.raises(ValueError, match="one device"):
        mat.triangle_attention(c.q, c.k.cpu(), c.v, c.bias, kv_lengths=c.kv_lengths)
    with pytest.raises(ValueError, match="one device"):
        mat.triangle_attention(c.q, c.k, c.v.cpu(), c.bias, kv_lengths=c.kv_lengths)
    out, lse, mx = mat.triangle_attention(c.q, c.k, c.v, c.bias, kv_lengths=c.kv_lengths,
                                          return_aux=True)
    with pytest.raises(ValueError, match="q's device"):
        mat.triangle_attention_backward(c.q, c.k, c.v, c.bias, out, out.cpu(), lse, mx,
                                        kv_lengths=c.kv_lengths)
    with pytest.raises(ValueError, match="q's device"):
        mat.triangle_attention_backward(c.q, c.k, c.v, c.bias, out, out, lse.cpu(), mx,
                                        kv_lengths=c.kv_lengths)
    q = torch.randn(40, 2, 32, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(40, 2, 32, dtype=torch.bfloat16)
    cu = torch.tensor([0, 15, 40], dtype=torch.int32)
    with pytest.raises(ValueError, match="one device"):
        mat.triangle_attention_varlen(q, k, k.cuda(), cu, cu, 25, 25)
    torch.cuda.synchronize()


def test_unaligned_views_are_copied_not_rejected():
    """Contiguous views at an offset that is not a multiple of 16 bytes give
    the same result as aligned copies of the same values."""
    say("unaligned input views")
    c = wl.make_case(1, 2, 2, 32, 32, 32, "bf16", "kv_lengths", seed=13).to("cuda")
    want = mat.triangle_attention(c.q, c.k, c.v, c.bias, kv_lengths=c.kv_lengths)
    def shifted(t):  # same values, 2 bytes past a 16-byte boundary
        buf = torch.empty(t.numel() + 8, device=t.device, dtype=t.dtype)
        view = buf[1:1 + t.numel()].view(t.shape)
        view.copy_(t)
        assert view.data_ptr() % 16 != 0
        return view
    got = mat.triangle_attention(shifted(c.q), shifted(c.k), shifted(c.v), c.bias,
                                 kv_lengths=c.kv_lengths)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


def test_four_d_inputs_and_side_stream():
    say("4-D inputs (B=1) on a side stream")
    c = wl.make_case(1, 3, 2, 80, 80, 64, "bf16", "kv_lengths", seed=11)
    ref = run_gpu(c)
    g = c.to("cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse, mx = mat.triangle_attention(g.q[0], g.k[0], g.v[0], g.bias[0],
                                              kv_lengths=g.kv_lengths[0], scale=g.scale,
                                              return_aux=True)
    s.synchronize()
    assert out.shape == g.q.shape[1:] and lse.shape == (3, 2, 80, 1)
    assert torch.equal(out.cpu(), ref[0][0]) and torch.equal(lse.cpu(), ref[1][0])


def test_mask_to_kv_lengths():
    say("mask_to_kv_lengths")
    lens = torch.tensor([0, 1, 5, 64, 100, 129, 130], dtype=torch.int32)
    K = 130
    mask = (torch.arange(K).view(1, 1, K) < lens.view(1, 7, 1)).view(1, 7, 1, 1, K)
    got = mat.mask_to_kv_lengths(mask.cuda())
    assert torch.equal(got.cpu().view(-1), lens)
    holey = mask.clone()
    holey[0, 3, 0, 0, 70] = True  # a valid key after the first masked one
    with pytest.raises(ValueError):
        mat.mask_to_kv_lengths(holey.cuda())
    got4 = mat.mask_to_kv_lengths(mask[0].cuda())
    assert got4.shape == (7, 1, 1, 1)


def test_blockmask_with_callable_causal_and_tuple_block_size():
    say("BlockMask causal callable")
    g = torch.Generator().manual_seed(12)
    c = wl.make_case(1, 1, 2, 256, 256, 64, "bf16", "none", seed=12, bias=False)
    lists = wl.causal_block_lists(g, 2, 128, 128)
    bm = mat.BlockMask.from_kv_blocks(lists.kv_num_blocks.cuda(), lists.kv_indices.cuda(),
                                      lists.full_kv_num_blocks.cuda(),
                                      lists.full_kv_indices.cuda(), BLOCK_SIZE=(128, 128),
                                      mask_mod=mat.causal_mask)
    gq = c.to("cuda")
    out = mat.triangle_attention(gq.q, gq.k, gq.v, None, block_mask=bm)
    ref = torch.nn.functional.scaled_dot_product_attention(
        c.q.float(), c.k.float(), c.v.float(), is_causal=True)
    assert (out.cpu().float() - ref).abs().max() < 2e-2


@pytest.mark.parametrize("B,N,H,Q,K,D,dt", [(1, 0, 2, 16, 8, 64, "bf16"), (1, 2, 2, 0, 8, 64, "f16"),
                                            (0, 2, 2, 16, 8, 32, "f32"), (1, 2, 0, 16, 8, 32, "bf16")])
def test_empty_work_returns_empty_outputs(B, N, H, Q, K, D, dt):
    """No query row: every mask kind returns outputs of the right (empty)
    shape and launches nothing; empty tensors hand over NULL addresses."""
    say(f"empty work B{B} N{N} H{H} Q{Q} K{K} D{D} {dt}")
    dtype = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
    q = torch.randn(B, N, H, Q, D, device="cuda").to(dtype)
    k = torch.randn(B, N, H, K, D, device="cuda").to(dtype)
    v = torch.randn(B, N, H, K, D, device="cuda").to(dtype)
    bias = torch.randn(B, 1, H, Q, K, device="cuda")
    lens = torch.full((B, N, 1, 1, 1), 3, device="cuda", dtype=torch.int32)
    mask = torch.ones(B, N, 1, 1, K, device="cuda", dtype=torch.bool)
    for kw in ({}, {"kv_lengths": lens}, {"mask": mask}):
        out, lse, mx = mat.triangle_attention(q, k, v, bias, return_aux=True, **kw)
        torch.cuda.synchronize()
        assert out.shape == q.shape and out.dtype == dtype
        assert lse.shape == (B, N, H, Q, 1) and mx.shape == (B, N, H, Q, 1)
    lens2 = mat.mask_to_kv_lengths(mask)
    assert lens2.shape == (B, N, 1, 1, 1)


def test_graph_capture_replays_match_eager():
    """tri_attn_fwd and tri_attn_bwd allocate nothing and launch only
    kernels, so they can be captured in a HIP graph: every replay, with eager
    work and synchronisations between replays, equals the eager result
    bitwise."""
    say("graph capture of forward and backward")
    c = wl.make_case(1, 4, 2, 96, 80, 64, "bf16", "kv_lengths", seed=41).to("cuda")
    dout = torch.randn(c.q.shape, generator=torch.Generator().manual_seed(43)).to(c.q.dtype).cuda()
    B, N, H, Q, K, D = c.shape
    desc = nat.TriAttnMask()
    desc.kind = nat.TRIATTN_MASK_KV_LENGTHS
    desc.kv_lengths = c.kv_lengths.data_ptr()
    shape = nat.TriAttnShape(B, N, H, Q, K, D)
    dt = nat.DTYPE_CODES[c.q.dtype]
    out, lse, mx = torch.empty_like(c.q), torch.empty(B, N, H, Q, device="cuda"), \
        torch.empty(B, N, H, Q, device="cuda")
    dq, dk, dv = torch.empty_like(c.q), torch.empty_like(c.k), torch.empty_like(c.v)
    db = torch.empty_like(c.bias)
    ws = torch.empty((mat.tri_attn_bwd_workspace_size(shape, True) + 3) // 4, device="cuda")

    def run(stream):
        assert mat.tri_attn_fwd(shape, dt, c.q, c.k, c.v, c.bias, desc, math.nan, out, lse, mx,
                                stream) == mat.TRIATTN_OK
        assert mat.tri_attn_bwd(shape, dt, c.q, c.k, c.v, c.bias, desc, math.nan, out, dout,
                                lse, mx, dq, dk, dv, db, stream, workspace=ws) == mat.TRIATTN_OK

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        run(side)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, lse, mx, dq, dk, dv, db)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run(side)
    for rep in range(3):
        for t in (out, lse, mx, dq, dk, dv, db):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = (out, lse, mx, dq, dk, dv, db)
        assert all(torch.equal(a, b) for a, b in zip(got, eager)), f"replay {rep} differs"
        torch.cuda.synchronize()
        _ = (c.q.float() * 2).sum().item()  # eager work between replays


def test_slices_past_32_bit_offsets():
    """K = 2^24 keys at D = 64 (each (b, n, h) slice of k and v is 2 GiB, so
    offsets pass 2^31 bytes): the library routes this to the kernel with
    64-bit addressing, and with every length at most 100 the result must
    equal the oracle on the first 100 keys alone (later keys never count)."""
    say("K = 2^24, D = 64, bf16, kv_lengths <= 100")
    B, N, H, Q, K, D = 1, 1, 2, 8, 1 << 24, 64
    g = torch.Generator(device="cuda").manual_seed(53)
    q = torch.randn(B, N, H, Q, D, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(B, N, H, K, D, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(B, N, H, K, D, device="cuda", generator=g).to(torch.bfloat16)
    lens = torch.tensor([77], dtype=torch.int32, device="cuda").view(1, 1, 1, 1, 1)
    out, lse, mx = mat.triangle_attention(q, k, v, None, kv_lengths=lens, return_aux=True)
    torch.cuda.synchronize()
    k100, v100 = k[:, :, :, :100].cpu(), v[:, :, :, :100].cpu()
    del k, v
    O, L, M = orc.oracle_fwd(q.cpu(), k100, v100, None, kv_lengths=lens.cpu(),
                             scale=1 / math.sqrt(D))
    assert np.abs(out.cpu().double().numpy() - O).max() <= TOL[torch.bfloat16]["o"]
    assert np.abs(lse.cpu().double().numpy().reshape(L.shape)
                  - L.astype(np.float32)).max() <= TOL[torch.bfloat16]["lse"]
    assert np.abs(mx.cpu().double().numpy().reshape(M.shape)
                  - M.astype(np.float32)).max() <= TOL[torch.bfloat16]["mx"]


def test_valid_logits_below_the_replacement_value():
    """The kernels carry masked logits as -inf, which equals the -1e9
    replacement whenever a valid logit exceeds -1e9 + 700.  This pins what
    they do in the case the two differ: a row whose every valid logit is far
    below -1e9 (bias -3e9).  The valid keys still take all the weight (here
    uniformly: in fp32, -3e9 + s.q.k rounds to -3e9), so O is the mean of V
    over the valid keys and max is -3e9, while the -1e9 replacement of the
    equation would average V over the masked keys instead."""
    say("valid logits below -1e9")
    B, N, H, Q, K, D = 1, 2, 2, 64, 96, 64
    c = wl.make_case(B, N, H, Q, K, D, "bf16", "dense", seed=31)
    c.bias[0, 0, 1, 5, :] = -3.0e9
    c.bias[0, 0, 0, 40, :] = -3.0e9
    out, lse, mx = run_gpu(c)
    valid = c.mask.view(B, N, K)
    for h, qrow in ((1, 5), (0, 40)):
        for n in range(N):
            vk = c.v[0, n, h].double()[valid[0, n]]
            want = vk.mean(dim=0)
            got = out[0, n, h, qrow].double()
            assert (got - want).abs().max() <= TOL[c.dtype]["o"], (h, qrow, n)
            assert float(mx[0, n, h, qrow]) == -3.0e9
            assert abs(float(lse[0, n, h, qrow]) + 3.0e9) <= 256.0
    # every other row is the equation's result
    rows = [i for i in range(B * N * H * Q)
            if (i // Q) % H != 1 or i % Q != 5]
    rows = [i for i in rows if (i // Q) % H != 0 or i % Q != 40]
    assert_parity(c, gpu=(out, lse, mx), rows=np.array(rows))
