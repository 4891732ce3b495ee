"""The no-allocation backward (tri_attn_bwd_noalloc) through the C ABI,
against tri_attn_bwd given a caller-owned workspace: both run the same
kernels on the same values, so every gradient must have the same bits.  Two
calls in a row, the second smaller, check that the library's shared scratch
(the per-row data) carries nothing over from one call to the next."""
import math

import pytest
import torch

import masked_attention_tri_amd as mat
from masked_attention_tri_amd import _native as nat
from masked_attention_tri_amd import workloads as wl
from tests.gpu_common import say

pytestmark = pytest.mark.gpu


def _backward(c, dout, noalloc):
    g = c.to("cuda")
    out, lse, mx = mat.triangle_attention(g.q, g.k, g.v, g.bias, mask=g.mask, scale=g.scale,
                                          return_aux=True, kv_lengths=g.kv_lengths)
    B, N, H, Q, K, D = c.shape
    desc, keep = None, []
    if g.mask is not None:
        m = g.mask.contiguous().view(torch.uint8)
        keep.append(m)
        desc = nat.TriAttnMask()
        desc.kind = nat.TRIATTN_MASK_DENSE
        desc.dense = m.data_ptr()
    elif g.kv_lengths is not None:
        desc = nat.TriAttnMask()
        desc.kind = nat.TRIATTN_MASK_KV_LENGTHS
        desc.kv_lengths = g.kv_lengths.data_ptr()
    dq, dk, dv = torch.empty_like(g.q), torch.empty_like(g.k), torch.empty_like(g.v)
    dbias = torch.empty(B, 1, H, Q, K, device="cuda")
    shp = nat.TriAttnShape(B, N, H, Q, K, D)
    dt = nat.DTYPE_CODES[g.q.dtype]
    s = math.nan if g.scale is None else g.scale
    args = (shp, dt, g.q, g.k, g.v, g.bias, desc, s, out, dout, lse, mx, dq, dk, dv, dbias)
    if noalloc:
        st = nat.tri_attn_bwd_noalloc(*args, None)
    else:
        ws = torch.empty((nat.tri_attn_bwd_workspace_size(shp, True) + 3) // 4, device="cuda")
        st = nat.tri_attn_bwd(*args, None, workspace=ws)
    torch.cuda.synchronize()
    assert st == mat.TRIATTN_OK, mat.tri_attn_status_str(st)
    return dq, dk, dv, dbias


@pytest.mark.parametrize("spec", [
    (1, 4, 2, 160, 160, 64, "bf16", "kv_lengths", {"len_range": (0, 160)}),
    # the second call is smaller: the first's row data must not leak into it
    (1, 2, 2, 96, 96, 32, "f16", "dense", {}),
])
def test_noalloc_backward_equals_workspace_backward(spec):
    B, N, H, Q, K, D, dt, kind, extra = spec
    c = wl.make_case(B, N, H, Q, K, D, dt, kind, seed=77, **extra)
    say(f"no-allocation backward {c.name}")
    dout = torch.randn(c.q.shape, generator=torch.Generator().manual_seed(78)).to(c.q.dtype)
    dout = dout.cuda()
    want = _backward(c, dout, noalloc=False)
    got = _backward(c, dout, noalloc=True)
    for name, a, b in zip(("dq", "dk", "dv", "dbias"), got, want):
        assert torch.equal(a, b), f"{name} differs"
    assert float(got[3].abs().max()) > 0
