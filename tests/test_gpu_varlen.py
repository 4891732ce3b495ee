"""GPU parity of the packed variable-length forward (Transformer Engine
fused_attn.h layouts: separate q/k/v, interleaved qkv, q with interleaved
kv; cu_seqlens offsets; PADDING / NO_MASK / CAUSAL) against the fp64 oracle.

The oracle is applied per sequence by a test-side split: sequence b's query
rows, key rows and heads become one (1, 1, H, Lq, D) / (1, 1, H, Lk, D)
problem without bias; the causal mask is one block covering the whole
sequence whose mask_mod is the causal predicate (q_idx >= kv_idx), which
the oracle evaluates element by element.  A sequence with no key rows has
no softmax at all: the library's documented value (O = 0, lse = max = -1e9)
is the expected one there.
"""
import math

import numpy as np
import pytest
import torch

import masked_attention_tri_amd as mat
import oracle as orc
from masked_attention_tri_amd import workloads as wl
from tests.gpu_common import TOL, say

pytestmark = pytest.mark.gpu


def _cu(lengths):
    return torch.tensor([0] + np.cumsum(lengths).tolist(), dtype=torch.int32)


def _draw(gen, rows, H, D, dtype, extra=()):
    return torch.randn(rows, *extra, H, D, generator=gen).to(wl.DTYPES[dtype])


def _oracle(q, k, v, cu_q, cu_kv, causal, scale, H, D, nq_max=None, nk_max=None):
    """(O, lse, max) per packed query row (rows of no sequence: NaN)."""
    Tq = q.shape[0]
    O = np.full((Tq, H, D), np.nan)
    L = np.full((Tq, H), np.nan)
    M = np.full((Tq, H), np.nan)
    for b in range(cu_q.numel() - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_kv[b]), int(cu_kv[b + 1])
        if nq_max is not None:
            q1 = min(q1, q0 + nq_max)
        if nk_max is not None:
            k1 = min(k1, k0 + nk_max)
        lq, lk = q1 - q0, k1 - k0
        if lq <= 0:
            continue
        if lk <= 0:
            O[q0:q1], L[q0:q1], M[q0:q1] = 0.0, -1.0e9, -1.0e9
            continue
        qb = q[q0:q1].permute(1, 0, 2).unsqueeze(0).unsqueeze(0)
        kb = k[k0:k1].permute(1, 0, 2).unsqueeze(0).unsqueeze(0)
        vb = v[k0:k1].permute(1, 0, 2).unsqueeze(0).unsqueeze(0)
        blk = None
        if causal:
            blk = orc.OracleBlockMask(np.array([[1]], dtype=np.int32),
                                      np.array([[[0]]], dtype=np.int32), q_block=lq,
                                      kv_block=lk, mask_mod=orc.MOD_CAUSAL)
        o, l, m = orc.oracle_fwd(qb, kb, vb, None, block=blk, scale=scale)
        O[q0:q1] = o[0, 0].transpose(1, 0, 2)
        L[q0:q1] = l[0, 0].T
        M[q0:q1] = m[0, 0].T
    return O, L, M


def _compare(got, want, dtype, name):
    go, gl, gm = (x.cpu().double().numpy() for x in got)
    O, L, M = want
    rows = ~np.isnan(L[:, 0])
    tol = TOL[dtype]
    eo = float(np.abs(go[rows] - O[rows]).max(initial=0.0))
    el = float(np.abs(gl[rows] - L[rows].astype(np.float32)).max(initial=0.0))
    em = float(np.abs(gm[rows] - M[rows].astype(np.float32)).max(initial=0.0))
    say(f"{name}: err O {eo:.3g} lse {el:.3g} max {em:.3g}")
    assert eo <= tol["o"] and el <= tol["lse"] and em <= tol["mx"], (eo, el, em)
    return rows


CASES = [
    # (layout, mask, dtype, H, D, q lengths, kv lengths)
    ("separate", "padding", "bf16", 3, 64, [37, 0, 130, 65, 200, 1], [40, 5, 129, 65, 256, 1]),
    ("separate", "causal", "bf16", 2, 64, [96, 33, 160], [96, 20, 200]),
    ("separate", "no_mask", "f16", 2, 128, [50, 129], [70, 31]),
    ("qkv_packed", "causal", "f16", 4, 32, [64, 1, 97, 300], None),
    ("qkv_packed", "padding", "bf16", 2, 64, [128, 77], None),
    ("kv_packed", "causal", "bf16", 2, 128, [40, 257, 3], [64, 200, 3]),
    ("kv_packed", "padding", "bf16", 3, 32, [10, 90], [300, 45]),
    # fp32 (the fp32 MFMA kernel): every layout, sequences past one 128-row
    # tile, an empty one; and head dimensions between the tile widths (the
    # MFMA kernel of the next width, zero columns)
    ("separate", "causal", "f32", 2, 32, [30, 17], [25, 40]),
    ("qkv_packed", "causal", "f32", 2, 16, [200, 1, 0, 129], None),
    ("kv_packed", "padding", "f32", 3, 28, [140, 60], [70, 300]),
    ("separate", "no_mask", "f32", 2, 8, [257, 5], [33, 0]),
    ("kv_packed", "padding", "bf16", 2, 40, [33, 64], [70, 12]),
    ("qkv_packed", "causal", "f16", 2, 136, [45, 20], None),
    ("separate", "no_mask", "bf16", 2, 96, [70, 200], [90, 33]),
]


@pytest.mark.parametrize("spec", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}-D{c[4]}" for c in CASES])
def test_varlen_matches_oracle_per_sequence(spec):
    layout, mask, dt, H, D, lq, lk = spec
    say(f"varlen {layout} {mask} {dt} H{H} D{D} q{lq} kv{lk}")
    gen = torch.Generator().manual_seed(sum(lq) * 7 + D)
    lk = lq if lk is None else lk
    Tq, Tk = sum(lq), sum(lk)
    cu_q, cu_kv = _cu(lq), _cu(lk)
    scale = 0.3 if mask == "no_mask" else None
    if layout == "qkv_packed":
        qkv = _draw(gen, Tq, H, D, dt, (3,))
        q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
        args = (qkv.cuda(), None, None, cu_q.cuda(), None)
    elif layout == "kv_packed":
        q = _draw(gen, Tq, H, D, dt)
        kv = _draw(gen, Tk, H, D, dt, (2,))
        k, v = kv[:, 0], kv[:, 1]
        args = (q.cuda(), kv.cuda(), None, cu_q.cuda(), cu_kv.cuda())
    else:
        q, k, v = _draw(gen, Tq, H, D, dt), _draw(gen, Tk, H, D, dt), _draw(gen, Tk, H, D, dt)
        args = (q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_kv.cuda())
    got = mat.triangle_attention_varlen(*args, max(lq), max(lk), layout=layout,
                                        mask_type=mask, scale=scale, return_aux=True)
    torch.cuda.synchronize()
    s = 1.0 / math.sqrt(D) if scale is None else scale
    want = _oracle(q, k, v, cu_q, cu_kv, mask == "causal", s, H, D)
    _compare(got, want, q.dtype, f"varlen {layout} {mask}")


def test_varlen_bounds_and_unwritten_rows():
    """Rows outside every sequence stay as they were; a sequence longer than
    max_seqlen is computed over its first max_seqlen rows (query and key);
    a key sequence of length 0 gives O = 0, lse = max = -1e9; and reversed
    or out-of-range offsets are clamped into the packed tensors."""
    say("varlen bounds")
    H, D, dt = 2, 64, "bf16"
    gen = torch.Generator().manual_seed(5)
    Tq, Tk = 400, 420
    q, k, v = _draw(gen, Tq, H, D, dt), _draw(gen, Tk, H, D, dt), _draw(gen, Tk, H, D, dt)
    # seq 0: 100 q rows / 80 keys; seq 1: q rows 100..299 (longer than the
    # bound 150) / 0 keys; seq 2: 60 q rows / 300 keys (longer than 150);
    # rows 360..399 of q belong to no sequence
    cu_q = torch.tensor([0, 100, 300, 360], dtype=torch.int32)
    cu_kv = torch.tensor([0, 80, 80, 380], dtype=torch.int32)
    d = mat.TriAttnVarlen()
    d.layout, d.mask_type = mat.TRIATTN_QKV_SEPARATE, mat.TRIATTN_VARLEN_PADDING
    d.batch, d.heads, d.head_dim, d.total_q, d.total_kv = 3, H, D, Tq, Tk
    gq, gk, gv, gcq, gck = (x.cuda() for x in (q, k, v, cu_q, cu_kv))
    d.cu_seqlens_q, d.cu_seqlens_kv = gcq.data_ptr(), gck.data_ptr()
    d.max_seqlen_q = d.max_seqlen_kv = 150
    out = torch.full((Tq, H, D), float("nan"), device="cuda").to(q.dtype)
    lse = torch.full((Tq, H), float("nan"), device="cuda")
    mx = torch.full((Tq, H), float("nan"), device="cuda")
    st = mat.tri_attn_varlen_fwd(d, mat.TRIATTN_BF16, gq, gk, gv, math.nan, out, lse, mx, None)
    torch.cuda.synchronize()
    assert st == mat.TRIATTN_OK
    want = _oracle(q, k, v, cu_q, cu_kv, False, 1 / math.sqrt(D), H, D, nq_max=150, nk_max=150)
    rows = _compare((out, lse, mx), want, q.dtype, "varlen bounds")
    written = torch.isfinite(lse.cpu()[:, 0]).numpy()
    assert (written == rows).all(), "rows written must be exactly the computed rows"
    assert rows[:100].all() and rows[100:250].all() and not rows[250:300].any()
    assert rows[300:360].all() and not rows[360:].any()
    assert torch.all(out.cpu()[100:250].float() == 0) and torch.all(mx.cpu()[100:250] == -1e9)
    # offsets past the tensors and reversed: clamped, nothing out of bounds
    bad = torch.tensor([0, 5000, 10, -7], dtype=torch.int32).cuda()
    d.cu_seqlens_q = bad.data_ptr()
    d.cu_seqlens_kv = bad.data_ptr()
    st = mat.tri_attn_varlen_fwd(d, mat.TRIATTN_BF16, gq, gk, gv, math.nan, out, lse, mx, None)
    torch.cuda.synchronize()
    assert st == mat.TRIATTN_OK
    assert torch.isfinite(out.float()[:150]).all()
