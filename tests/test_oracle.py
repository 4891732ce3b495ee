"""The fp64 oracle against its pins (CPU only).

See tests/oracle_pins.py for what pins which part of the definition.
"""
import numpy as np
import pytest

import oracle as orc
from masked_attention_tri_amd import workloads as wl
from tests import helpers as hp
from tests import oracle_pins as pins


@pytest.mark.parametrize("name,check", pins.ALL_CHECKS, ids=[n for n, _ in pins.ALL_CHECKS])
def test_oracle_pin(name, check):
    check(orc.oracle_fwd)


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_oracle_library_random_seeds(seed):
    for c in pins.library_cases(seed=seed):
        pins.check_against_library(orc.oracle_fwd, c)


def test_oracle_small_workloads_against_library():
    # fp32 with a dense all-ones mask, and fp16 with kv_lengths = 96
    for key in ("fp32_dense_ones", "fp16_lens96"):
        pins.check_against_library(orc.oracle_fwd, wl.make_workload(key))


def test_oracle_dense_half_rows_against_library():
    # the bf16 dense-mask workload restricted to a few n rows, including the four fully masked ones
    c = wl.make_workload("bf16_dense_half")
    keep = sorted(set(c.meta["fully_masked_rows"]) | {0, 1, 200, 383})
    sub = wl.Case(c.name, c.dtype, c.q[:, keep], c.k[:, keep], c.v[:, keep], c.bias,
                  mask=c.mask[:, keep], scale=c.scale)
    pins.check_against_library(orc.oracle_fwd, sub)


def test_oracle_causal_blocks_rows_against_causal_library():
    # the block workload's lists are causal; sampled q rows against is_causal on b=0,h=0
    import torch
    import torch.nn.functional as F

    c = wl.make_workload("bf16_causal_blocks_d128")
    qs = [0, 1, 127, 128, 129, 2047, 4095]
    rows = [q for q in qs]  # b = 0, n = 0, h = 0
    O, lse, mx = hp.run_oracle(c, rows=rows)
    q = c.q[0, 0, 0].double()
    k = c.k[0, 0, 0].double()
    v = c.v[0, 0, 0].double()
    s = 1.0 / np.sqrt(128)
    for i, qi in enumerate(qs):
        logits = (q[qi] @ k[: qi + 1].T) * s
        w = torch.softmax(logits, dim=0)
        ref = w @ v[: qi + 1]
        assert np.abs(O[i] - ref.numpy()).max() < 1e-10
    ref_full = F.scaled_dot_product_attention(q[None, None, :130], k[None, None], v[None, None],
                                              attn_mask=torch.ones(130, 4096, dtype=torch.bool)
                                              .tril())
    assert np.abs(O[:5] - ref_full[0, 0, [0, 1, 127, 128, 129]].numpy()).max() < 1e-10


def test_oracle_rejects_bad_arguments():
    c = wl.make_case(1, 1, 1, 2, 2, 4, "f32", "none")
    with pytest.raises(ValueError):
        orc.oracle_fwd(c.q, c.k, c.v, c.bias, mask=np.ones((1, 1, 2)),
                       kv_lengths=np.ones((1, 1)))
    with pytest.raises(RuntimeError):
        orc.oracle_fwd(c.q, c.k, c.v, c.bias, rows=[4])
