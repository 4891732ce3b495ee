"""Property tests of the fp64 oracle over tiny random shapes (CPU only).

Each property follows from the definition on the triangle_attention page
(the softmax attention over keys with an additive pair bias and the -1e9
replacement of masked logits, returning O, lse and max) and the BlockMask
page (block lists as a key mask), not from how the oracle computes it:

* relabelling keys (K, V, bias columns and mask together) changes nothing;
* a constant added to one query row's bias shifts that row's lse and max by
  it and leaves O unchanged;
* O is affine in V (the weights sum to one), and lies inside the range of
  the valid keys' V (inside all keys' V for a row with none);
* max <= lse <= max + ln(number of valid keys);
* the three mask forms agree when they describe the same key set, lengths
  past K clamp to K and lengths <= 0 mask every key;
* the scale multiplies Q.K only, and defaults to 1/sqrt(D);
* a row subset returns exactly the full evaluation's rows;
* backward: dV summed over keys equals dO summed over queries (every row's
  weights sum to one), and each query row of dBias sums to zero over keys
  (the softmax Jacobian's rows do), with zeros at masked keys.
"""
import math

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as orc

SETTINGS = dict(max_examples=100, deadline=None, database=None,
                suppress_health_check=[HealthCheck.too_slow])
TOL = 1e-10


@st.composite
def problems(draw, mask_kinds=("none", "dense", "kv_lengths")):
    B = draw(st.integers(1, 2))
    N = draw(st.integers(1, 3))
    H = draw(st.integers(1, 2))
    Q = draw(st.integers(1, 5))
    K = draw(st.integers(1, 7))
    D = draw(st.integers(1, 5))
    seed = draw(st.integers(0, 2**31 - 1))
    kind = draw(st.sampled_from(mask_kinds))
    with_bias = draw(st.booleans())
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, H, Q, D))
    k = rng.standard_normal((B, N, H, K, D))
    v = rng.standard_normal((B, N, H, K, D))
    bias = 2.0 * rng.standard_normal((B, 1, H, Q, K)) if with_bias else None
    mask = lens = None
    if kind == "dense":
        mask = rng.random((B, N, K)) < 0.6
        if draw(st.booleans()):
            mask[0, 0, :] = False  # a row n with no valid key
    elif kind == "kv_lengths":
        lens = rng.integers(-1, K + 2, size=(B, N)).astype(np.int32)
    scale = draw(st.sampled_from([None, 0.25, 0.7, 1.0]))
    return dict(q=q, k=k, v=v, bias=bias, mask=mask, lens=lens, scale=scale)


def run(p, **over):
    a = dict(p)
    a.update(over)
    return orc.oracle_fwd(a["q"], a["k"], a["v"], a["bias"], mask=a["mask"],
                          kv_lengths=a["lens"], scale=a["scale"])


def valid_keys(p):
    """(B, N, K) bool: the keys each row n may attend to."""
    B, N, _, _, _ = p["q"].shape
    K = p["k"].shape[3]
    if p["mask"] is not None:
        return p["mask"].astype(bool)
    if p["lens"] is not None:
        return np.arange(K)[None, None, :] < np.clip(p["lens"], 0, K)[:, :, None]
    return np.ones((B, N, K), dtype=bool)


def close(a, b, tol=TOL):
    np.testing.assert_allclose(a, b, rtol=tol, atol=tol)


@settings(**SETTINGS)
@given(problems(mask_kinds=("none", "dense")), st.randoms(use_true_random=False))
def test_key_relabelling_changes_nothing(p, rnd):
    K = p["k"].shape[3]
    perm = list(range(K))
    rnd.shuffle(perm)
    perm = np.array(perm)
    O, lse, mx = run(p)
    O2, lse2, mx2 = run(p, k=p["k"][:, :, :, perm], v=p["v"][:, :, :, perm],
                        bias=None if p["bias"] is None else p["bias"][..., perm],
                        mask=None if p["mask"] is None else p["mask"][..., perm])
    close(O, O2)
    close(lse, lse2)
    close(mx, mx2)


@settings(**SETTINGS)
@given(problems(), st.floats(-30.0, 30.0))
def test_row_bias_constant_shifts_lse_and_max_only(p, c):
    B, N, H, Q, _ = p["q"].shape
    K = p["k"].shape[3]
    bias = p["bias"] if p["bias"] is not None else np.zeros((B, 1, H, Q, K))
    shift = np.zeros((B, 1, H, Q, 1))
    shift[..., 0, 0] = c  # query row 0 of every (b, h)
    O, lse, mx = run(p, bias=bias)
    O2, lse2, mx2 = run(p, bias=bias + shift)
    live = valid_keys(p).any(-1)[:, :, None, None]  # rows n with a valid key
    expect = np.where(live, shift[:, :, :, :, 0], 0.0)  # (B, N|1, H, Q)
    close(O, O2, 1e-9)
    close(lse2 - lse, np.broadcast_to(expect, lse.shape), 1e-9)
    close(mx2 - mx, np.broadcast_to(expect, mx.shape), 1e-9)


@settings(**SETTINGS)
@given(problems(), st.floats(-3.0, 3.0), st.floats(-5.0, 5.0))
def test_output_is_affine_in_v(p, alpha, beta):
    O, lse, mx = run(p)
    O2, lse2, mx2 = run(p, v=alpha * p["v"] + beta)
    close(O2, alpha * O + beta, 1e-9)
    close(lse, lse2)
    close(mx, mx2)


@settings(**SETTINGS)
@given(problems())
def test_output_in_valid_value_range_and_lse_bounds(p):
    O, lse, mx = run(p)
    ok = valid_keys(p)  # (B, N, K)
    v = p["v"]
    B, N, H, Q, D = O.shape
    for b in range(B):
        for n in range(N):
            keys = ok[b, n]
            sel = keys if keys.any() else np.ones_like(keys)
            for h in range(H):
                lo = v[b, n, h][sel].min(0)
                hi = v[b, n, h][sel].max(0)
                assert np.all(O[b, n, h] >= lo - 1e-12) and np.all(O[b, n, h] <= hi + 1e-12)
                if keys.any():
                    m = mx[b, n, h]
                    assert np.all(lse[b, n, h] >= m - 1e-12)
                    assert np.all(lse[b, n, h] <= m + math.log(keys.sum()) + 1e-12)
                else:
                    # the -1e9 replacement: uniform weights over all K keys
                    assert np.all(mx[b, n, h] == -1e9)
                    close(lse[b, n, h], -1e9 + math.log(ok.shape[-1]))


@settings(**SETTINGS)
@given(problems(mask_kinds=("kv_lengths",)))
def test_mask_forms_agree(p):
    B, N, H, Q, _ = p["q"].shape
    K = p["k"].shape[3]
    lens = p["lens"]
    dense = np.arange(K)[None, None, :] < np.clip(lens, 0, K)[:, :, None]
    # one query block of Q rows, one key per kv block, a list per (b, n, h)
    cnt = np.repeat(np.clip(lens, 0, K).reshape(B * N, 1), H, axis=1).reshape(B * N * H, 1)
    idx = np.tile(np.arange(K, dtype=np.int32), (B * N * H, 1, 1))
    blk = orc.OracleBlockMask(cnt.astype(np.int32), idx, q_block=Q, kv_block=1,
                              stride_b=N * H, stride_n=H, stride_h=1)
    a = run(p)
    b = run(p, lens=None, mask=dense)
    c = orc.oracle_fwd(p["q"], p["k"], p["v"], p["bias"], block=blk, scale=p["scale"])
    for x, y, z in zip(a, b, c):
        close(x, y, 0.0)
        close(x, z, 0.0)


@settings(**SETTINGS)
@given(problems(mask_kinds=("none",)), st.integers(0, 3))
def test_lengths_clamp(p, extra):
    B, N = p["q"].shape[:2]
    K = p["k"].shape[3]
    full = run(p)
    past = run(p, lens=np.full((B, N), K + extra, dtype=np.int32))
    for x, y in zip(full, past):
        close(x, y, 0.0)
    none = run(p, lens=np.full((B, N), -extra, dtype=np.int32))
    mean_v = np.broadcast_to(p["v"].mean(3, keepdims=True), full[0].shape)
    close(none[0], mean_v)
    assert np.all(none[2] == -1e9)


@settings(**SETTINGS)
@given(problems(), st.sampled_from([0.125, 0.3, 1.7]))
def test_scale_multiplies_qk_only(p, s):
    a = run(p, scale=s)
    b = run(p, q=p["q"] * s, scale=1.0)
    for x, y in zip(a, b):
        close(x, y, 1e-9)
    D = p["q"].shape[-1]
    for x, y in zip(run(p, scale=None), run(p, scale=1.0 / math.sqrt(D))):
        close(x, y, 0.0)


@settings(**SETTINGS)
@given(problems(), st.randoms(use_true_random=False))
def test_row_subset_matches_full(p, rnd):
    O, lse, mx = run(p)
    n_rows = lse.size
    rows = sorted(rnd.sample(range(n_rows), min(n_rows, 4)))
    a = orc.oracle_fwd(p["q"], p["k"], p["v"], p["bias"], mask=p["mask"],
                       kv_lengths=p["lens"], scale=p["scale"], rows=rows)
    close(a[0], O.reshape(n_rows, -1)[rows], 0.0)
    close(a[1], lse.reshape(-1)[rows], 0.0)
    close(a[2], mx.reshape(-1)[rows], 0.0)


@settings(**dict(SETTINGS, max_examples=50))
@given(problems(), st.integers(0, 2**31 - 1))
def test_backward_sums(p, seed):
    dout = np.random.default_rng(seed).standard_normal(p["q"].shape)
    bias = p["bias"]
    if bias is None:
        B, _, H, Q, _ = p["q"].shape
        bias = np.zeros((B, 1, H, Q, p["k"].shape[3]))
    dq, dk, dv, db = orc.oracle_bwd(p["q"], p["k"], p["v"], bias, dout=dout, mask=p["mask"],
                                    kv_lengths=p["lens"], scale=p["scale"])
    # every row's weights sum to one: sum_k dV_k = sum_q dO_q per (b, n, h)
    close(dv.sum(3), dout.sum(3), 1e-9)
    # softmax Jacobian rows sum to zero; masked keys get no bias gradient
    close(db.sum(-1), np.zeros(db.shape[:-1]), 1e-9)
    ok = valid_keys(p)  # (B, N, K)
    # a key masked in every row n has no gradient in any (b, h, q)
    never = ~ok.any(1)  # (B, K)
    assert np.all(db[:, 0][np.broadcast_to(never[:, None, None, :], db[:, 0].shape)] == 0.0)
