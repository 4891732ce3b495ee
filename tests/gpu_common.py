"""Shared helpers of the GPU tests: run the library on a Case, compare with
the fp64 oracle at the specified tolerances."""
from __future__ import annotations

import numpy as np
import torch

import masked_attention_tri_amd as mat
from tests import helpers as hp

# O max-abs against the unrounded fp64 oracle; lse and max against the
# oracle rounded to fp32.  fp32: 1e-5 for all three; fp16/bf16: 2e-2 on O,
# 1e-3 on lse and max.
TOL = {
    torch.float32: dict(o=1e-5, lse=1e-5, mx=1e-5),
    torch.float16: dict(o=2e-2, lse=1e-3, mx=1e-3),
    torch.bfloat16: dict(o=2e-2, lse=1e-3, mx=1e-3),
}


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def block_mask_of(case):
    b = case.block
    if b is None:
        return None
    return mat.BlockMask.from_kv_blocks(b.kv_num_blocks, b.kv_indices, b.full_kv_num_blocks,
                                        b.full_kv_indices, BLOCK_SIZE=(b.kv_block, b.q_block),
                                        mask_mod=b.mask_mod)


def mask_descriptor(case):
    """(TriAttnMask descriptor, objects it points into) of a device Case,
    built by the package's own argument preparation."""
    prep = mat._prepare(case.q, case.k, case.v, case.bias, case.mask, case.kv_lengths,
                        block_mask_of(case))
    return prep[5], prep


def run_gpu(case, stream=None, scale="case"):
    """(O, lse, max) from the library, copied to the CPU."""
    c = case.to("cuda")
    s = c.scale if scale == "case" else scale
    out = mat.triangle_attention(c.q, c.k, c.v, c.bias, mask=c.mask, scale=s, return_aux=True,
                                 kv_lengths=c.kv_lengths, block_mask=block_mask_of(c),
                                 stream=stream)
    torch.cuda.synchronize()
    return tuple(x.cpu() for x in out)


def errors(case, gpu, rows=None, oracle=None):
    """Max-abs errors (O, lse, max) of the GPU result against the oracle."""
    O, lse, mx = oracle if oracle is not None else hp.run_oracle(case, rows=rows)
    D = case.shape[5]
    go = gpu[0].double().reshape(-1, D).numpy()
    gl = gpu[1].double().reshape(-1).numpy()
    gm = gpu[2].double().reshape(-1).numpy()
    if rows is not None:
        go, gl, gm = go[rows], gl[rows], gm[rows]
    O = np.asarray(O).reshape(-1, D)
    lse32 = np.asarray(lse, dtype=np.float64).reshape(-1).astype(np.float32).astype(np.float64)
    mx32 = np.asarray(mx, dtype=np.float64).reshape(-1).astype(np.float32).astype(np.float64)
    assert np.isfinite(go).all() and np.isfinite(gl).all() and np.isfinite(gm).all(), \
        "non-finite output"
    return (float(np.abs(go - O).max(initial=0.0)), float(np.abs(gl - lse32).max(initial=0.0)),
            float(np.abs(gm - mx32).max(initial=0.0)))


def assert_parity(case, gpu=None, rows=None, oracle=None):
    gpu = gpu if gpu is not None else run_gpu(case)
    eo, el, em = errors(case, gpu, rows=rows, oracle=oracle)
    tol = TOL[case.dtype]
    say(f"{case.name}: err O {eo:.3g} lse {el:.3g} max {em:.3g}")
    assert eo <= tol["o"], f"{case.name}: O error {eo} > {tol['o']}"
    assert el <= tol["lse"], f"{case.name}: lse error {el} > {tol['lse']}"
    assert em <= tol["mx"], f"{case.name}: max error {em} > {tol['mx']}"
    return eo, el, em
