"""Pins of the fp64 oracle to things other than itself.

Each check takes ``fwd`` (an oracle_fwd-compatible callable) so the same
checks can run against the real oracle and against deliberately broken
copies of it (tests/test_oracle_mutants.py).  A check raises AssertionError
on a mismatch.

What pins what (definition: the triangle_attention page's equation, its
"scale" / "mask" / "kv_lengths" parameter notes, and the BlockMask format of
the tensorplay.nn.attention page):
  * golden worked examples, derived by hand as closed forms (tests/golden);
  * torch's scaled_dot_product_attention in float64 on the CPU, a library
    routine: O for rows with a valid key, with the float attn_mask
    bias + (-inf on masked keys) added after scaling, as in the equation;
  * lse through the same library routine: one extra key with logit 0 and a
    one-hot value column receives weight w = 1 / (1 + e^lse), so
    lse = log((1 - w) / w);
  * max through the library's attention weights (identity values):
    max_k w_k = exp(max - lse);
  * closed forms: K = 1, q = 0 (uniform weights), constant bias, fully masked
    rows (uniform over all K keys, max = -1e9, lse = -1e9 + ln K);
  * invariants: per-row bias shift, key permutation, convex hull of V,
    default scale, kv_lengths clamps, kv_lengths == prefix dense mask,
    block lists == dense reconstruction, full lists are only an
    optimisation, causal lists == the library's is_causal.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from masked_attention_tri_amd import workloads as wl
from tests import helpers as hp

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NEG = -1.0e9


def _sdpa(case, valid, extra=None):
    """Library attention in float64 with masked keys at -inf."""
    B, N, H, Q, K, D = case.shape
    q = case.q.double()
    k = case.k.double()
    v = case.v.double()
    bias = case.bias.double().expand(B, N, H, Q, K) if case.bias is not None \
        else torch.zeros(B, N, H, Q, K, dtype=torch.float64)
    am = bias.masked_fill(~valid, float("-inf"))
    if extra is not None:
        k, v, am = extra(k, v, am)
    s = case.scale if case.scale is not None else 1.0 / math.sqrt(D)
    return F.scaled_dot_product_attention(q, k, v, attn_mask=am, scale=s)


def _sink(k, v, am):
    """Append one key with q.k = 0, logit 0 and value e_D (a new column)."""
    B, N, H, K, D = k.shape
    Q = am.shape[3]
    k2 = torch.cat([k, torch.zeros(B, N, H, 1, D, dtype=k.dtype)], dim=3)
    v2 = torch.zeros(B, N, H, K + 1, D + 1, dtype=v.dtype)
    v2[..., :K, :D] = v
    v2[..., K, D] = 1.0
    am2 = torch.cat([am, torch.zeros(B, N, H, Q, 1, dtype=am.dtype)], dim=4)
    return k2, v2, am2


def _onehot(k, v, am):
    K = k.shape[3]
    eye = torch.eye(K, dtype=v.dtype).expand(*v.shape[:3], K, K).contiguous()
    return k, eye, am


def check_against_library(fwd, case, o_tol=1e-10, lse_tol=1e-9):
    """O, lse and max against torch SDPA (float64) for rows with a valid key;
    closed form (uniform over all K, -1e9) for rows with none."""
    O, lse, mx = hp.run_oracle(case, fwd=fwd)
    O, lse, mx = torch.from_numpy(O), torch.from_numpy(lse), torch.from_numpy(mx)
    valid = hp.valid_matrix(case)
    has = valid.any(dim=-1)
    ref = _sdpa(case, valid)
    if has.any():
        err = (O - ref)[has].abs().max().item()
        assert err <= o_tol, f"O vs library attention: {err}"
        w = _sdpa(case, valid, extra=_sink)[..., -1]
        lse_lib = torch.log1p(-w) - torch.log(w)
        err = (lse - lse_lib)[has].abs().max().item()
        assert err <= lse_tol, f"lse vs library attention: {err}"
        W = _sdpa(case, valid, extra=_onehot)
        mx_lib = lse_lib + torch.log(W.max(dim=-1).values)
        err = (mx - mx_lib)[has].abs().max().item()
        assert err <= lse_tol, f"max vs library attention weights: {err}"
    dead = ~has
    if dead.any():
        K = case.shape[4]
        meanv = case.v.double().mean(dim=3, keepdim=True).expand_as(O)
        err = (O - meanv)[dead].abs().max().item()
        assert err <= 1e-12, f"fully masked row O != mean V: {err}"
        assert torch.all(mx[dead] == NEG), "fully masked row max != -1e9"
        err = (lse[dead] - (NEG + math.log(K))).abs().max().item()
        assert err <= 1e-6, f"fully masked row lse: {err}"


def check_golden(fwd):
    files = sorted(f for f in os.listdir(GOLDEN) if f.startswith("worked_"))
    assert files, "no golden worked examples found"
    env = {"log": math.log, "exp": math.exp, "sqrt": math.sqrt, "e": math.e,
           "__builtins__": {}}

    def ev(x):
        if isinstance(x, list):
            return [ev(y) for y in x]
        if isinstance(x, str):
            return float(eval(x, env))
        return x

    for fn in files:
        with open(os.path.join(GOLDEN, fn)) as f:
            g = json.load(f)
        for ex in g["examples"]:
            inp = ex["inputs"]
            args = dict(q=np.array(ev(inp["q"]), dtype=np.float64),
                        k=np.array(ev(inp["k"]), dtype=np.float64),
                        v=np.array(ev(inp["v"]), dtype=np.float64))
            bias = np.array(ev(inp["bias"]), dtype=np.float64) \
                if inp.get("bias") is not None else None
            kw = {"scale": inp.get("scale")}
            if "mask" in inp:
                kw["mask"] = np.array(inp["mask"], dtype=np.uint8)
            if "kv_lengths" in inp:
                kw["kv_lengths"] = np.array(inp["kv_lengths"], dtype=np.int32)
            if "block" in inp:
                import oracle as orc

                bl = inp["block"]
                kw["block"] = orc.OracleBlockMask(
                    np.array(bl["kv_num_blocks"], dtype=np.int32),
                    np.array(bl["kv_indices"], dtype=np.int32),
                    None if bl.get("full_kv_num_blocks") is None
                    else np.array(bl["full_kv_num_blocks"], dtype=np.int32),
                    None if bl.get("full_kv_indices") is None
                    else np.array(bl["full_kv_indices"], dtype=np.int32),
                    q_block=bl["q_block"], kv_block=bl["kv_block"],
                    mask_mod=1 if bl.get("mask_mod") == "causal" else 0)
            O, lse, mx = fwd(args["q"], args["k"], args["v"], bias, **kw)
            exp_o = np.array(ev(ex["expect"]["O"]))
            exp_l = np.array(ev(ex["expect"]["lse"]))
            exp_m = np.array(ev(ex["expect"]["max"]))
            tol = ex.get("tol", 1e-12)
            name = f"{fn}:{ex['name']}"
            assert np.allclose(O.reshape(exp_o.shape), exp_o, rtol=0, atol=tol), \
                f"{name}: O {O.reshape(-1)} != {exp_o.reshape(-1)}"
            assert np.allclose(lse.reshape(-1), exp_l, rtol=1e-15, atol=tol), \
                f"{name}: lse {lse.reshape(-1)} != {exp_l}"
            assert np.allclose(mx.reshape(-1), exp_m, rtol=1e-15, atol=tol), \
                f"{name}: max {mx.reshape(-1)} != {exp_m}"


def check_closed_forms(fwd, seed=0):
    # K = 1: the single key gets weight 1, so O = V_0 and lse = max.
    c = wl.make_case(2, 2, 2, 5, 1, 8, "f32", "none", seed=seed)
    O, lse, mx = hp.run_oracle(c, fwd=fwd)
    assert np.array_equal(O, c.v.double().expand(2, 2, 2, 5, 8).numpy()), "K=1: O != V0"
    assert np.allclose(lse, mx, rtol=0, atol=1e-15), "K=1: lse != max"
    # q = 0 and bias = c per (b,h,q): uniform weights over the valid keys.
    for kind in ("none", "dense", "kv_lengths"):
        c = wl.make_case(2, 3, 2, 4, 11, 8, "f32", kind, seed=seed + 1, len_range=(1, 11))
        c.q = torch.zeros_like(c.q)
        const = torch.randn(2, 1, 2, 4, 1, generator=torch.Generator().manual_seed(seed))
        c.bias = const.expand(2, 1, 2, 4, 11).contiguous()
        O, lse, mx = hp.run_oracle(c, fwd=fwd)
        valid = hp.valid_matrix(c).double()
        cnt = valid.sum(-1)
        vv = c.v.double()
        mean_valid = (valid.unsqueeze(-1) * vv.unsqueeze(3)).sum(4) / cnt.unsqueeze(-1).clamp(min=1)
        has = cnt > 0
        assert np.allclose(O[has.numpy()], mean_valid[has].numpy(), rtol=0, atol=1e-12), \
            f"{kind}: uniform weights"
        cc = const.expand(2, 3, 2, 4, 1)[..., 0]
        assert np.allclose(mx[has.numpy()], cc[has].numpy(), rtol=0, atol=1e-15), \
            f"{kind}: max != constant bias"
        assert np.allclose(lse[has.numpy()], (cc + torch.log(cnt))[has].numpy(), rtol=0,
                           atol=1e-12), f"{kind}: lse != c + ln(count)"


def check_invariants(fwd, seed=0):
    c = wl.make_case(2, 2, 3, 9, 13, 16, "bf16", "dense", seed=seed, bias_sigma=2.0,
                     scale=0.37)
    O, lse, mx = hp.run_oracle(c, fwd=fwd)
    # a constant added to a bias row moves max and lse by it, O unchanged
    shift = torch.randn(2, 1, 3, 9, 1, generator=torch.Generator().manual_seed(seed + 7)) * 3
    c2 = wl.Case(c.name, c.dtype, c.q, c.k, c.v, (c.bias.double() + shift), mask=c.mask,
                 scale=c.scale)
    O2, lse2, mx2 = hp.run_oracle(c2, fwd=fwd)
    sh = shift[..., 0].expand(2, 2, 3, 9).numpy()
    has = hp.valid_matrix(c).any(-1).numpy()
    assert np.allclose(O2[has], O[has], rtol=0, atol=1e-12), "bias shift changed O"
    assert np.allclose(mx2[has], (mx + sh)[has], rtol=0, atol=1e-12), "bias shift: max"
    assert np.allclose(lse2[has], (lse + sh)[has], rtol=0, atol=1e-12), "bias shift: lse"
    # permuting keys consistently (k, v, bias columns, mask) changes nothing
    perm = torch.randperm(13, generator=torch.Generator().manual_seed(seed + 3))
    c3 = wl.Case(c.name, c.dtype, c.q, c.k[:, :, :, perm], c.v[:, :, :, perm],
                 c.bias[..., perm], mask=c.mask[..., perm], scale=c.scale)
    O3, lse3, mx3 = hp.run_oracle(c3, fwd=fwd)
    assert np.allclose(O3, O, rtol=0, atol=1e-12), "key permutation changed O"
    assert np.allclose(lse3, lse, rtol=0, atol=1e-12), "key permutation changed lse"
    assert np.array_equal(mx3, mx), "key permutation changed max"
    # every output lies in the convex hull of the valid values
    valid = hp.valid_matrix(c)
    vv = c.v.double().unsqueeze(3).expand(2, 2, 3, 9, 13, 16)
    vmask = valid.unsqueeze(-1).expand_as(vv)
    hi = vv.masked_fill(~vmask, -np.inf).max(dim=4).values.numpy()
    lo = vv.masked_fill(~vmask, np.inf).min(dim=4).values.numpy()
    assert np.all(O[has] <= hi[has] + 1e-12) and np.all(O[has] >= lo[has] - 1e-12), "hull"
    # default scale is 1/sqrt(D), exactly
    c4 = wl.make_case(1, 2, 2, 6, 7, 16, "f16", "none", seed=seed + 4)
    a = hp.run_oracle(c4, fwd=fwd, scale=None)
    b = hp.run_oracle(c4, fwd=fwd, scale=1.0 / math.sqrt(16))
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "scale=None != 1/sqrt(D)"


def check_kv_lengths(fwd, seed=0):
    c = wl.make_case(2, 5, 2, 6, 9, 8, "f16", "kv_lengths", seed=seed, len_range=(0, 9))
    c.kv_lengths = torch.tensor([0, 1, 4, 8, 9, 3, 9, 2, 5, 7], dtype=torch.int32).view(
        2, 5, 1, 1, 1)
    base = hp.run_oracle(c, fwd=fwd)
    # a prefix dense mask of L ones is the same mask
    dense = torch.arange(9).view(1, 1, 1, 1, 9) < c.kv_lengths
    cd = wl.Case(c.name, c.dtype, c.q, c.k, c.v, c.bias, mask=dense, scale=c.scale)
    for x, y in zip(base, hp.run_oracle(cd, fwd=fwd)):
        assert np.array_equal(x, y), "kv_lengths != prefix dense mask"
    # values above K clamp to K; values below 0 read as 0
    cl = wl.Case(c.name, c.dtype, c.q, c.k, c.v, c.bias,
                 kv_lengths=torch.where(c.kv_lengths == 9, 14, torch.where(
                     c.kv_lengths == 0, -3, c.kv_lengths)).to(torch.int32), scale=c.scale)
    for x, y in zip(base, hp.run_oracle(cl, fwd=fwd)):
        assert np.array_equal(x, y), "kv_lengths clamps"
    check_against_library(fwd, c)


def check_blocks(fwd, seed=0):
    # random lists (shuffled, duplicates, out-of-range ids, full blocks some of
    # which the kv list does not name) against the dense reconstruction
    for mod in ("none", "causal"):
        c = wl.make_case(2, 2, 2, 40, 37, 8, "bf16", "block", seed=seed + (mod == "causal"),
                         q_block=16, kv_block=8, mask_mod=mod)
        check_against_library(fwd, c)
    cb = wl.make_case(1, 3, 2, 24, 24, 8, "f32", "block", seed=seed + 5, q_block=8,
                      kv_block=8, mask_mod="causal", block_broadcast=True)
    check_against_library(fwd, cb)
    # causal lists (as in the block-sparse workload) equal the library's is_causal
    g = torch.Generator().manual_seed(seed + 9)
    c = wl.make_case(1, 1, 2, 64, 64, 16, "bf16", "none", seed=seed + 9, bias=False)
    c.block = wl.causal_block_lists(g, 4, 16, 16)
    O, lse, mx = hp.run_oracle(c, fwd=fwd)
    ref = F.scaled_dot_product_attention(c.q.double(), c.k.double(), c.v.double(),
                                         is_causal=True)
    err = np.abs(O - ref.numpy()).max()
    assert err <= 1e-10, f"causal lists vs is_causal: {err}"
    # full lists are purely an optimisation: dropping them (the kv lists still
    # name every block) must not change anything
    c_nf = wl.Case(c.name, c.dtype, c.q, c.k, c.v, None,
                   block=wl.BlockLists(c.block.kv_num_blocks, c.block.kv_indices, None, None,
                                       16, 16, "causal"))
    for x, y in zip((O, lse, mx), hp.run_oracle(c_nf, fwd=fwd)):
        assert np.array_equal(x, y), "full_kv lists changed the result"


def check_rows_and_threads(fwd, seed=0):
    c = wl.make_case(2, 3, 2, 7, 10, 8, "bf16", "kv_lengths", seed=seed)
    O, lse, mx = hp.run_oracle(c, fwd=fwd, threads=1)
    O3, lse3, mx3 = hp.run_oracle(c, fwd=fwd, threads=3)
    assert np.array_equal(O, O3) and np.array_equal(lse, lse3) and np.array_equal(mx, mx3)
    rows = np.array([0, 83, 5, 41, 41, 12])
    Or, lr, mr = hp.run_oracle(c, fwd=fwd, rows=rows)
    assert np.array_equal(Or, O.reshape(-1, 8)[rows])
    assert np.array_equal(lr, lse.reshape(-1)[rows])
    assert np.array_equal(mr, mx.reshape(-1)[rows])


def library_cases(seed=0):
    """Random cases that together cover every mask kind, dtype and odd shape."""
    return [
        wl.make_case(2, 3, 2, 9, 13, 8, "f32", "none", seed=seed),
        wl.make_case(1, 4, 3, 12, 7, 16, "bf16", "dense", seed=seed + 1, bias_sigma=2.0),
        wl.make_case(2, 4, 2, 5, 17, 24, "f16", "kv_lengths", seed=seed + 2, scale=0.29),
        wl.make_case(2, 2, 2, 33, 31, 8, "bf16", "block", seed=seed + 3, q_block=8,
                     kv_block=16, mask_mod="causal"),
        wl.make_case(1, 2, 2, 6, 6, 4, "f32", "dense", seed=seed + 4, p_valid=0.15),
    ]


ALL_CHECKS = [
    ("golden", lambda fwd: check_golden(fwd)),
    ("library", lambda fwd: [check_against_library(fwd, c) for c in library_cases()]),
    ("closed_forms", lambda fwd: check_closed_forms(fwd)),
    ("invariants", lambda fwd: check_invariants(fwd)),
    ("kv_lengths", lambda fwd: check_kv_lengths(fwd)),
    ("blocks", lambda fwd: check_blocks(fwd)),
    ("rows_threads", lambda fwd: check_rows_and_threads(fwd)),
]
