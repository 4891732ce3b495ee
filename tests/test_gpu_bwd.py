"""GPU parity of the backward pass (dQ, dK, dV, dBias) against the fp64
backward oracle.

Each case runs the library's forward (O, lse, max), then its backward with a
seeded incoming gradient dO, and compares every gradient element with the
oracle's exact gradient of the same inputs.  Tolerance: the kernels
accumulate in fp32 (for the half types, P and dz enter the MFMAs rounded to
the input type) and round dq, dk and dv once to the input type; the oracle
is exact.  For the half types the rounding alone is up to 2^-8 of the
largest value (bf16), and Delta = dO . O inherits the forward's rounded O,
so the bound is 2e-2 of the tensor's largest magnitude (plus 2e-2
absolute); for fp32, 1e-4 of it (plus 1e-4).  dbias is fp32 for every input type and gets the
same bound as its input type's gradients.
"""
import numpy as np
import pytest
import torch

import masked_attention_tri_amd as mat
import oracle as orc
from masked_attention_tri_amd import workloads as wl
from tests import helpers as hp
from tests.gpu_common import block_mask_of, say

pytestmark = pytest.mark.gpu

REL = {torch.float32: 1e-4, torch.float16: 2e-2, torch.bfloat16: 2e-2}


def _oracle_bwd(c, dout):
    kw = {}
    if c.mask is not None:
        kw["mask"] = c.mask
    elif c.kv_lengths is not None:
        kw["kv_lengths"] = c.kv_lengths
    elif c.block is not None:
        kw["block"] = hp.oracle_block(c)
    return orc.oracle_bwd(c.q, c.k, c.v, c.bias, dout=dout, scale=c.scale, **kw)


def _check(c, seed):
    g = torch.Generator().manual_seed(seed)
    dout = torch.randn(c.q.shape, generator=g).to(c.q.dtype)
    gc = c.to("cuda")
    bm = block_mask_of(gc)
    out, lse, mx = mat.triangle_attention(gc.q, gc.k, gc.v, gc.bias, mask=gc.mask,
                                          scale=gc.scale, return_aux=True,
                                          kv_lengths=gc.kv_lengths, block_mask=bm)
    grads = mat.triangle_attention_backward(gc.q, gc.k, gc.v, gc.bias, out, dout.cuda(), lse,
                                            mx, mask=gc.mask, scale=gc.scale,
                                            kv_lengths=gc.kv_lengths, block_mask=bm)
    torch.cuda.synchronize()
    ref = _oracle_bwd(c, dout)
    rel = REL[c.q.dtype]
    for name, got, want in zip(("dq", "dk", "dv", "dbias"), grads, ref):
        if want is None:
            assert got is None, name
            continue
        got = got.cpu().double().numpy()
        assert np.isfinite(got).all(), f"{c.name} {name}: non-finite"
        err = float(np.abs(got - want).max(initial=0.0))
        bound = rel * (1.0 + float(np.abs(want).max(initial=0.0)))
        say(f"{c.name} {name}: err {err:.3g} bound {bound:.3g}")
        assert err <= bound, f"{c.name} {name}: error {err} > {bound}"


CASES = [
    # (B, N, H, Q, K, D, dtype, kind, extra)
    (1, 2, 2, 40, 37, 32, "f32", "kv_lengths", {"len_range": (-2, 45)}),
    (1, 3, 2, 33, 50, 64, "bf16", "dense", {}),
    (2, 2, 2, 70, 65, 64, "bf16", "kv_lengths", {}),
    (1, 2, 2, 64, 96, 128, "f16", "none", {}),
    (1, 2, 2, 30, 40, 40, "bf16", "dense", {"p_valid": 0.05}),
    (2, 1, 2, 64, 64, 32, "bf16", "block", {"q_block": 16, "kv_block": 16, "mask_mod": "causal"}),
    (1, 2, 2, 48, 48, 64, "f16", "none", {"bias": False, "scale": 0.3}),
    (1, 2, 2, 20, 30, 256, "bf16", "kv_lengths", {}),
    (1, 2, 2, 16, 1, 32, "f32", "none", {}),
    # register-resident MFMA kernels: ragged Q and K past 128, many rows with
    # no valid key (lengths <= 0) and tiny lengths
    (1, 6, 2, 130, 200, 64, "bf16", "kv_lengths", {"len_range": (-3, 3)}),
    # D = 32, K not a multiple of 4 (scalar dz and dBias paths), about half
    # the rows fully masked
    (1, 3, 2, 40, 130, 32, "f16", "dense", {"p_valid": 0.005}),
    # 32- and 64-row query blocks on the MFMA kernels (dQ: 4 or 2 block rows
    # per workgroup): non-causal, causal with full lists and a ragged last
    # block row, sparse lists (rows with no listed block), D = 32 / 64 / 128
    (1, 2, 2, 96, 96, 64, "bf16", "block", {"q_block": 32, "kv_block": 32}),
    (1, 2, 2, 200, 230, 128, "bf16", "block", {"q_block": 64, "kv_block": 32, "mask_mod": "causal"}),
    (1, 2, 2, 160, 128, 32, "f16", "block", {"q_block": 32, "kv_block": 64, "block_density": 0.3}),
    (2, 1, 2, 256, 256, 64, "bf16", "block", {"q_block": 32, "kv_block": 32, "mask_mod": "causal",
                                               "block_broadcast": True, "bias": False}),
    # dBias of block lists on the MFMA kernel: lists per n, several n ranges
    # summed by the combine kernel
    (1, 8, 2, 256, 200, 64, "bf16", "block", {"q_block": 64, "kv_block": 64, "mask_mod": "causal"}),
    (1, 6, 1, 130, 260, 128, "f16", "block", {"q_block": 128, "kv_block": 32,
                                              "block_density": 0.4}),
    # MFMA kernels: causal block lists (partial diagonal blocks, unlisted and
    # full blocks) with a bias
    (1, 2, 2, 256, 256, 64, "bf16", "block", {"q_block": 128, "kv_block": 64, "mask_mod": "causal"}),
    # D = 128, sparse lists: query blocks with no listed block (rows without a
    # valid key), several kv blocks per 128-key workgroup
    (1, 2, 2, 384, 200, 128, "f16", "block", {"q_block": 128, "kv_block": 32,
                                              "block_density": 0.25}),
    (1, 2, 2, 200, 160, 128, "bf16", "kv_lengths", {}),
    (2, 3, 2, 100, 72, 32, "bf16", "dense", {}),
    # scale that is not a power of two; K % 4 != 0 (per-lane bias loads)
    (1, 2, 2, 96, 70, 64, "bf16", "none", {"scale": 0.3}),
    # s = 0: z is the bias alone
    (1, 3, 2, 64, 64, 64, "f16", "kv_lengths", {"scale": 0.0}),
    # head dimensions between the tile widths (zero columns on the next width)
    (1, 3, 2, 130, 150, 96, "bf16", "kv_lengths", {"len_range": (0, 150)}),
    (1, 2, 2, 100, 90, 24, "f16", "dense", {}),
    (1, 2, 2, 256, 256, 48, "bf16", "block", {"q_block": 128, "kv_block": 64, "mask_mod": "causal"}),
    (1, 2, 2, 70, 70, 72, "bf16", "none", {"scale": 0.3}),
    (1, 2, 2, 64, 64, 120, "f16", "kv_lengths", {"scale": 0.0}),
    (1, 3, 2, 40, 40, 8, "bf16", "kv_lengths", {}),
    (1, 48, 2, 128, 128, 40, "bf16", "kv_lengths", {}),  # dBias in ranges of n
]


@pytest.mark.parametrize("spec", CASES, ids=[f"B{c[0]}N{c[1]}H{c[2]}Q{c[3]}K{c[4]}D{c[5]}-{c[6]}-{c[7]}"
                                              for c in CASES])
def test_backward_matches_oracle(spec):
    B, N, H, Q, K, D, dt, kind, extra = spec
    c = wl.make_case(B, N, H, Q, K, D, dt, kind, seed=17, **extra)
    say(f"backward {c.name}")
    _check(c, seed=23)


def test_backward_workload_kv_lengths_fp16():
    """The fp16 kv_lengths workload (B1 N128 H2 Q=K=128 D32, lengths 96)."""
    c = wl.make_workload("fp16_lens96")
    say(f"backward {c.name}")
    _check(c, seed=29)


@pytest.mark.parametrize("four_d", [False, True])
def test_autograd_wrapper(four_d):
    """torch.autograd through triangle_attention_autograd gives the oracle's
    gradients of sum(O * G); 4-D (B = 1) inputs keep their rank."""
    c = wl.make_case(1, 2, 2, 40, 50, 64, "bf16", "kv_lengths", seed=31)
    say(f"autograd {c.name} four_d={four_d}")
    g = torch.Generator().manual_seed(37)
    dout = torch.randn(c.q.shape, generator=g).to(c.q.dtype)
    sq = (lambda t: t.squeeze(0)) if four_d else (lambda t: t)
    q, k, v = (sq(x).cuda().requires_grad_() for x in (c.q, c.k, c.v))
    bias = sq(c.bias).cuda().requires_grad_()
    lens = sq(c.kv_lengths).cuda()
    out = mat.triangle_attention_autograd(q, k, v, bias, kv_lengths=lens, scale=c.scale)
    assert out.shape == q.shape
    out.backward(sq(dout).cuda())
    ref = orc.oracle_bwd(c.q, c.k, c.v, c.bias, dout=dout, kv_lengths=c.kv_lengths, scale=c.scale)
    for name, t, want in zip(("dq", "dk", "dv", "dbias"), (q, k, v, bias), ref):
        got = t.grad.detach().cpu().double().reshape(want.shape).numpy()
        err = float(np.abs(got - want).max())
        bound = 2e-2 * (1 + float(np.abs(want).max()))
        say(f"autograd {name}: err {err:.3g} bound {bound:.3g}")
        assert err <= bound, f"{name}: {err} > {bound}"


def test_autograd_with_bias_in_input_dtype():
    """With the bias cast to the input type, autograd's gradients are those
    of the fp32 path given the rounded bias, bit for bit (the forward widens
    each 16-bit bias value exactly and the backward receives the same
    values); dbias comes back in the bias's own dtype."""
    c = wl.make_case(1, 3, 2, 64, 96, 64, "bf16", "kv_lengths", seed=43)
    say(f"autograd half bias {c.name}")
    g = torch.Generator().manual_seed(41)
    dout = torch.randn(c.q.shape, generator=g).to(c.q.dtype).cuda()
    grads = []
    for half in (True, False):
        q, k, v = (x.cuda().requires_grad_() for x in (c.q, c.k, c.v))
        b = (c.bias if half else c.bias.to(c.dtype).float()).cuda().requires_grad_()
        out = mat.triangle_attention_autograd(q, k, v, b, kv_lengths=c.kv_lengths.cuda(),
                                              scale=c.scale, bias_in_input_dtype=half)
        out.backward(dout)
        torch.cuda.synchronize()
        grads.append([out.detach()] + [t.grad for t in (q, k, v, b)])
    for name, a, r in zip(("out", "dq", "dk", "dv", "dbias"), *grads):
        assert torch.equal(a, r), name
    assert grads[0][4].dtype == torch.float32


def test_backward_headline_size_sampled():
    """The headline workload at full size (B1 N768 H4 Q=K=768 D64, bf16,
    kv_lengths): the GPU backward of every slice, with dQ, dK and dV of the
    first two n compared element by element with the oracle run on those
    slices alone (each (b, n, h) slice's dQ, dK, dV depend only on that
    slice; dBias, a sum over all n, is checked on the smaller cases)."""
    c = wl.make_workload("bf16_lens_d64")
    say(f"backward sampled {c.name}")
    g = torch.Generator().manual_seed(47)
    dout = torch.randn(c.q.shape, generator=g).to(c.q.dtype)
    gc = c.to("cuda")
    out, lse, mx = mat.triangle_attention(gc.q, gc.k, gc.v, gc.bias, scale=gc.scale,
                                          return_aux=True, kv_lengths=gc.kv_lengths)
    dq, dk, dv, _ = mat.triangle_attention_backward(gc.q, gc.k, gc.v, gc.bias, out, dout.cuda(),
                                                    lse, mx, scale=gc.scale,
                                                    kv_lengths=gc.kv_lengths)
    torch.cuda.synchronize()
    ns = 2
    ref = orc.oracle_bwd(c.q[:, :ns], c.k[:, :ns], c.v[:, :ns], c.bias, dout=dout[:, :ns],
                         kv_lengths=c.kv_lengths[:, :ns], scale=c.scale)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        got = got[:, :ns].cpu().double().numpy()
        err = float(np.abs(got - want).max())
        bound = 2e-2 * (1 + float(np.abs(want).max()))
        say(f"headline sampled {name}: err {err:.3g} bound {bound:.3g}")
        assert err <= bound, f"{name}: {err} > {bound}"


def _run_bwd(c, dout, ws_fill):
    """tri_attn_bwd through the C ABI with a workspace prefilled with ws_fill."""
    import masked_attention_tri_amd._native as nat
    from tests.gpu_common import mask_descriptor

    gc = c.to("cuda")
    bm = block_mask_of(gc)
    out, lse, mx = mat.triangle_attention(gc.q, gc.k, gc.v, gc.bias, mask=gc.mask,
                                          scale=gc.scale, return_aux=True,
                                          kv_lengths=gc.kv_lengths, block_mask=bm)
    B, N, H, Q, K, D = c.shape
    shape = nat.TriAttnShape(B, N, H, Q, K, D)
    ws = torch.full(((mat.tri_attn_bwd_workspace_size(shape, True) + 3) // 4,), ws_fill,
                    device="cuda", dtype=torch.float32)
    dq, dk, dv = torch.empty_like(gc.q), torch.empty_like(gc.k), torch.empty_like(gc.v)
    db = torch.empty_like(gc.bias) if gc.bias is not None else None
    desc, keep = mask_descriptor(gc)
    s = float("nan") if gc.scale is None else float(gc.scale)
    st = mat.tri_attn_bwd(shape, nat.DTYPE_CODES[gc.q.dtype], gc.q, gc.k, gc.v, gc.bias, desc, s,
                          out.reshape(gc.q.shape), dout, lse, mx, dq, dk, dv, db, None,
                          workspace=ws)
    torch.cuda.synchronize()
    assert st == mat.TRIATTN_OK, mat.tri_attn_status_str(st)
    return dq, dk, dv, db


@pytest.mark.parametrize("spec", CASES[1:4] + CASES[-7:],
                         ids=[f"B{c[0]}N{c[1]}H{c[2]}Q{c[3]}K{c[4]}D{c[5]}-{c[6]}-{c[7]}"
                              for c in CASES[1:4] + CASES[-7:]])
def test_backward_independent_of_workspace_contents(spec):
    """The workspace's contents on entry do not matter (every entry a later
    pass reads is written by the first), and the backward is deterministic:
    a NaN-filled and a zeroed workspace give the same bits."""
    B, N, H, Q, K, D, dt, kind, extra = spec
    c = wl.make_case(B, N, H, Q, K, D, dt, kind, seed=19, **extra)
    say(f"workspace contents {c.name}")
    g = torch.Generator().manual_seed(59)
    dout = torch.randn(c.q.shape, generator=g).to(c.q.dtype).cuda()
    a = _run_bwd(c, dout, float("nan"))
    b = _run_bwd(c, dout, 0.0)
    for name, x, y in zip(("dq", "dk", "dv", "dbias"), a, b):
        if x is None:
            continue
        assert torch.equal(x, y), f"{c.name} {name}: depends on the workspace's contents"


def test_dbias_split_matches_unsplit_headline():
    """At the headline size dBias sums over 768 n in ranges added in order
    (the workspace holds one plane of partial sums per extra range); with
    only the minimal workspace (the row data) the sum runs in one range.
    dq, dk and dv do not depend on it (same bits); dbias agrees to fp32
    rounding."""
    import masked_attention_tri_amd._native as nat

    c = wl.make_workload("bf16_lens_d64")
    say(f"dbias split {c.name}")
    B, N, H, Q, K, D = c.shape
    shape = nat.TriAttnShape(B, N, H, Q, K, D)
    full = mat.tri_attn_bwd_workspace_size(shape, True)
    least = mat.tri_attn_bwd_workspace_size(shape, False)
    assert full > least
    g = torch.Generator().manual_seed(73)
    dout = torch.randn(c.q.shape, generator=g).to(c.q.dtype).cuda()
    gc = c.to("cuda")
    out, lse, mx = mat.triangle_attention(gc.q, gc.k, gc.v, gc.bias, scale=gc.scale,
                                          return_aux=True, kv_lengths=gc.kv_lengths)
    desc, keep = __import__("tests.gpu_common", fromlist=["mask_descriptor"]).mask_descriptor(gc)
    res = []
    for size in (full, least):
        ws = torch.empty((size + 3) // 4, device="cuda")
        grads = [torch.empty_like(gc.q), torch.empty_like(gc.k), torch.empty_like(gc.v),
                 torch.empty_like(gc.bias)]
        st = mat.tri_attn_bwd(shape, nat.DTYPE_CODES[gc.q.dtype], gc.q, gc.k, gc.v, gc.bias, desc,
                              float(gc.scale), out, dout, lse, mx, *grads, None, workspace=ws)
        torch.cuda.synchronize()
        assert st == mat.TRIATTN_OK
        res.append(grads)
    for name, a, b in zip(("dq", "dk", "dv"), res[0][:3], res[1][:3]):
        assert torch.equal(a, b), name
    d = (res[0][3] - res[1][3]).abs().max().item()
    ref = res[1][3].abs().max().item()
    say(f"dbias split vs one range: max diff {d:.3g}, max |dbias| {ref:.3g}")
    assert d <= 1e-5 * ref


def test_block_causal_backward_config_shape():
    """The causal BlockMask workload at full size (B2 N1 H8 Q=K=4096 D128,
    128 x 128 blocks, bf16, no bias) through the MFMA backward: dQ of 24
    rows of every (b, h) (both ends of several 128-row tiles) against the
    oracle evaluated on those rows only, and dK, dV of two whole slices
    (b, h) = (0, 0) and (1, 7) against the oracle run on those slices."""
    c = wl.make_workload("bf16_causal_blocks_d128")
    say(f"backward block causal {c.name}")
    g = torch.Generator().manual_seed(71)
    dout = torch.randn(c.q.shape, generator=g).to(c.q.dtype)
    gc = c.to("cuda")
    bm = block_mask_of(gc)
    out, lse, mx = mat.triangle_attention(gc.q, gc.k, gc.v, None, return_aux=True,
                                          block_mask=bm)
    dq, dk, dv, _ = mat.triangle_attention_backward(gc.q, gc.k, gc.v, None, out, dout.cuda(),
                                                    lse, mx, block_mask=bm)
    torch.cuda.synchronize()
    blk = hp.oracle_block(c)
    qs = sorted({0, 1, 127, 128, 255, 1023, 1024, 2047, 2048, 2049, 3071, 3072, 4095}
                | set(torch.randperm(4096, generator=g)[:11].tolist()))
    ref = orc.oracle_bwd(c.q, c.k, c.v, None, dout=dout, block=blk, q_rows=qs)
    got = dq.cpu().double().numpy()[:, :, :, qs]
    want = ref[0][:, :, :, qs]
    err = float(np.abs(got - want).max())
    bound = 2e-2 * (1 + float(np.abs(want).max()))
    say(f"block causal dq ({len(qs)} rows x 16 slices): err {err:.3g} bound {bound:.3g}")
    assert err <= bound
    for b, h in ((0, 0), (1, 7)):
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        r = orc.oracle_bwd(c.q[sl], c.k[sl], c.v[sl], None, dout=dout[sl], block=blk)
        for name, t, want in (("dq", dq, r[0]), ("dk", dk, r[1]), ("dv", dv, r[2])):
            got = t[sl].cpu().double().numpy()
            err = float(np.abs(got - want).max())
            bound = 2e-2 * (1 + float(np.abs(want).max()))
            say(f"block causal ({b},{h}) {name}: err {err:.3g} bound {bound:.3g}")
            assert err <= bound, f"({b},{h}) {name}: {err} > {bound}"


def test_dbias_headline_size_against_oracle():
    """dBias at the headline size (B1 N768 H4 Q=K=768 D64, bf16, kv_lengths
    U{384..768}) against the fp64 backward oracle on 12 query rows of every
    head, each summed over all 768 n: the oracle evaluates only those rows
    (each row's gradient terms are independent of the others)."""
    c = wl.make_workload("bf16_lens_d64")
    say(f"dbias vs oracle {c.name}")
    g = torch.Generator().manual_seed(67)
    dout = torch.randn(c.q.shape, generator=g).to(c.q.dtype)
    gc = c.to("cuda")
    out, lse, mx = mat.triangle_attention(gc.q, gc.k, gc.v, gc.bias, scale=gc.scale,
                                          return_aux=True, kv_lengths=gc.kv_lengths)
    _, _, _, db = mat.triangle_attention_backward(gc.q, gc.k, gc.v, gc.bias, out, dout.cuda(),
                                                  lse, mx, scale=gc.scale,
                                                  kv_lengths=gc.kv_lengths)
    torch.cuda.synchronize()
    qs = sorted(set(torch.randperm(768, generator=g)[:10].tolist()) | {0, 767})
    ref = orc.oracle_bwd(c.q, c.k, c.v, c.bias, dout=dout, kv_lengths=c.kv_lengths,
                         scale=c.scale, q_rows=qs)[3]
    got = db.cpu().double().numpy()[:, :, :, qs]
    want = ref[:, :, :, qs]
    err = np.abs(got - want)
    scale_row = np.abs(want).max(axis=-1, keepdims=True)
    worst = float((err / scale_row).max())
    say(f"dbias headline: max abs err {float(err.max()):.3g}, max |ref| "
        f"{float(np.abs(want).max()):.3g}, worst err / row max {worst:.3g}")
    assert worst <= 2e-2, f"dbias error {worst} of the row's largest value"
