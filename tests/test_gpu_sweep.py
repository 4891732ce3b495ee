"""Seeded random sweep of the forward and the backward against the oracle.

The fixed-shape parity tests name the cases each kernel path was built for;
this sweep draws shapes, dtypes, head dimensions (every multiple of 8 up to
256 for the 16-bit types: the tile widths and the widths between them),
mask kinds (dense, lengths with both clamps, block lists of several block
sizes with and without the causal mask_mod), bias or none and scales from a
fixed seed, so that combinations nobody listed are checked too.  Every case
is compared element by element with the fp64 oracle at the same tolerances
as the other parity tests.
"""
import random

import pytest

from masked_attention_tri_amd import workloads as wl
from tests.gpu_common import assert_parity, say
from tests.test_gpu_bwd import _check

pytestmark = pytest.mark.gpu


def _specs(n, seed, max_d_half, max_qk):
    r = random.Random(seed)
    out = []
    for i in range(n):
        dt = r.choice(["bf16", "f16", "bf16", "f32"])
        D = r.choice([4, 8, 16, 24, 32]) if dt == "f32" else 8 * r.randint(1, max_d_half // 8)
        kind = r.choice(["none", "dense", "kv_lengths", "block"])
        B, N, H = r.randint(1, 2), r.randint(1, 3), r.randint(1, 2)
        Q, K = r.randint(1, max_qk), r.randint(1, max_qk)
        extra = {}
        if kind == "block":
            extra.update(q_block=r.choice([128, 128, 64, 32, 16]), kv_block=r.choice([32, 64, 128, 16]),
                         mask_mod=r.choice(["none", "causal"]))
        elif kind == "dense":
            extra["p_valid"] = r.choice([0.02, 0.5, 0.9])
        if r.random() < 0.25:
            extra["bias"] = False
        if r.random() < 0.3:
            extra["scale"] = r.choice([0.3, 0.125, 1.0, 0.0])
        out.append((B, N, H, Q, K, D, dt, kind, extra, 1000 + i))
    return out


def _id(s):
    B, N, H, Q, K, D, dt, kind, extra, seed = s
    return f"B{B}N{N}H{H}Q{Q}K{K}D{D}-{dt}-{kind}-s{seed}"


FWD = _specs(40, 20261203, 256, 300)
BWD = _specs(20, 20261204, 128, 160)


@pytest.mark.parametrize("spec", FWD, ids=[_id(s) for s in FWD])
def test_forward_sweep(spec):
    B, N, H, Q, K, D, dt, kind, extra, seed = spec
    c = wl.make_case(B, N, H, Q, K, D, dt, kind, seed=seed, **extra)
    say(f"sweep {c.name} {extra}")
    assert_parity(c)


@pytest.mark.parametrize("spec", BWD, ids=[_id(s) for s in BWD])
def test_backward_sweep(spec):
    B, N, H, Q, K, D, dt, kind, extra, seed = spec
    c = wl.make_case(B, N, H, Q, K, D, dt, kind, seed=seed, **extra)
    say(f"backward sweep {c.name} {extra}")
    _check(c, seed=seed + 1)
