"""Pins of the fp64 backward oracle (CPU only).

The backward oracle is checked against the forward oracle, not against
itself: central finite differences of L = sum(O * G) with respect to every
element of q, k, v and the bias, for every mask kind, must equal the
oracle's gradient for the incoming gradient G.  Closed forms cover one key
and rows with no valid key, and plausible mistakes planted in copies of the
backward oracle must fail these pins.
"""
import functools
import os

import numpy as np
import pytest

import oracle as orc
from oracle import oracle as orc_mod


def _case(kind, B=1, N=2, H=2, Q=3, K=5, D=4, bias=True, seed=0):
    g = np.random.default_rng(seed)
    c = dict(q=g.standard_normal((B, N, H, Q, D)), k=g.standard_normal((B, N, H, K, D)),
             v=g.standard_normal((B, N, H, K, D)),
             bias=g.standard_normal((B, 1, H, Q, K)) if bias else None,
             dout=g.standard_normal((B, N, H, Q, D)), scale=0.7, mk={})
    if kind == "dense":
        m = g.random((B, N, K)) < 0.6
        m[0, 1, :] = False  # one row (b=0, n=1) with no valid key
        c["mk"] = dict(mask=m)
    elif kind == "kv_lengths":
        c["mk"] = dict(kv_lengths=np.array([[3, 0]][:B], dtype=np.int32)[:, :N])
    elif kind == "block":
        # two query blocks of 2 rows, three kv blocks of 2 keys; causal on
        # the partial blocks, block 0 full for the second row of blocks
        nb = np.array([[1, 2]], dtype=np.int32)
        ix = np.array([[[0, 2], [1, 0]]], dtype=np.int32)
        fnb = np.array([[0, 1]], dtype=np.int32)
        fix = np.array([[[0, 0], [0, 0]]], dtype=np.int32)
        c["mk"] = dict(block=orc.OracleBlockMask(nb, ix, fnb, fix, q_block=2, kv_block=2,
                                                 mask_mod=orc.MOD_CAUSAL))
    return c


def _loss(c, fwd=orc.oracle_fwd, **over):
    args = {key: c[key] for key in ("q", "k", "v", "bias")}
    args.update(over)
    o, _, _ = fwd(args["q"], args["k"], args["v"], args["bias"], scale=c["scale"], **c["mk"])
    return float(np.sum(o * c["dout"]))


def _fd_grad(c, name, eps=1e-6):
    x = c[name]
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += eps
        xm[i] -= eps
        g[i] = (_loss(c, **{name: xp}) - _loss(c, **{name: xm})) / (2 * eps)
    return g


def _check_fd(c, bwd):
    dq, dk, dv, db = bwd(c["q"], c["k"], c["v"], c["bias"], dout=c["dout"], scale=c["scale"],
                         **c["mk"])
    for name, got in (("q", dq), ("k", dk), ("v", dv), ("bias", db)):
        if c[name] is None:
            assert got is None
            continue
        ref = _fd_grad(c, name)
        assert np.abs(got - ref).max() <= 1e-6 * (1 + np.abs(ref).max()), name


KINDS = ["none", "dense", "kv_lengths", "block"]


@pytest.mark.parametrize("kind", KINDS)
def test_gradient_matches_finite_differences(kind):
    _check_fd(_case(kind), orc.oracle_bwd)


def test_gradient_without_bias_and_default_scale():
    c = _case("dense", bias=False, seed=3)
    c["scale"] = None
    dq, dk, dv, db = orc.oracle_bwd(c["q"], c["k"], c["v"], None, dout=c["dout"], **c["mk"])
    assert db is None
    c["scale"] = 1 / np.sqrt(4)
    dq2, dk2, dv2, _ = orc.oracle_bwd(c["q"], c["k"], c["v"], None, dout=c["dout"],
                                      scale=c["scale"], **c["mk"])
    assert np.array_equal(dq, dq2) and np.array_equal(dk, dk2) and np.array_equal(dv, dv2)
    _check_fd(c, orc.oracle_bwd)


def test_one_key_closed_form():
    """K = 1: O = V_0 whatever the logits, so only V has a gradient: the sum
    of dO over the query rows."""
    c = _case("none", K=1, seed=5)
    dq, dk, dv, db = orc.oracle_bwd(c["q"], c["k"], c["v"], c["bias"], dout=c["dout"],
                                    scale=c["scale"])
    assert not dq.any() and not dk.any() and not db.any()
    assert np.allclose(dv[..., 0, :], c["dout"].sum(axis=3), atol=1e-12)


def test_rows_without_valid_key():
    """A row with no valid key averages V with weight 1/K: dV_k += dO/K and
    nothing reaches q, k or the bias."""
    c = _case("kv_lengths", N=1, seed=7)
    c["mk"] = dict(kv_lengths=np.array([[0]], dtype=np.int32))
    dq, dk, dv, db = orc.oracle_bwd(c["q"], c["k"], c["v"], c["bias"], dout=c["dout"],
                                    scale=c["scale"], **c["mk"])
    K = c["k"].shape[3]
    assert not dq.any() and not dk.any() and not db.any()
    want = np.repeat(c["dout"].sum(axis=3, keepdims=True) / K, K, axis=3)
    assert np.allclose(dv, want, atol=1e-12)


def test_bias_gradient_sums_over_n():
    """The bias is shared by every n: its gradient is the sum of the per-n
    gradients (each n alone, as an N = 1 problem)."""
    c = _case("dense", N=3, seed=9)
    c["mk"] = dict(mask=np.random.default_rng(1).random((1, 3, 5)) < 0.7)
    _, _, _, db = orc.oracle_bwd(c["q"], c["k"], c["v"], c["bias"], dout=c["dout"],
                                 scale=c["scale"], **c["mk"])
    parts = []
    for n in range(3):
        sl = slice(n, n + 1)
        _, _, _, dbn = orc.oracle_bwd(c["q"][:, sl], c["k"][:, sl], c["v"][:, sl], c["bias"],
                                      dout=c["dout"][:, sl], scale=c["scale"],
                                      mask=c["mk"]["mask"][:, sl])
        parts.append(dbn)
    assert np.allclose(db, sum(parts), atol=1e-12)


# ---- planted mistakes ----------------------------------------------------

MUTANTS = [
    ("no_delta", "const double dz = z[kk] * (dp[kk] - delta);",
     "const double dz = z[kk] * dp[kk];"),
    ("delta_sign", "const double dz = z[kk] * (dp[kk] - delta);",
     "const double dz = z[kk] * (dp[kk] + delta);"),
    ("dq_no_scale", "dqr[d] += a->scale * dz * kb[kk * D + d];", "dqr[d] += dz * kb[kk * D + d];"),
    ("dk_uses_v", "dkb[kk * D + d] += a->scale * dz * qr[d];",
     "dkb[kk * D + d] += a->scale * dz * vb[kk * D + d];"),
    ("dv_unnormalised", "for (int64_t kk = 0; kk < K; ++kk) z[kk] /= l;", "(void)l;"),
    ("dbias_last_n_only",
     "    double *dbias = a->dbias ? a->dbias + (b * H + h) * Q * K : NULL;\n"
     "    if (dbias) memset(dbias, 0, (size_t)(Q * K) * sizeof(double));\n"
     "    for (int64_t n = 0; n < N; ++n) {\n",
     "    double *dbias = a->dbias ? a->dbias + (b * H + h) * Q * K : NULL;\n"
     "    for (int64_t n = 0; n < N; ++n) {\n"
     "        if (dbias) memset(dbias, 0, (size_t)(Q * K) * sizeof(double));\n"),
    ("additive_mask", "z[kk] = -1.0e9;", "z[kk] = -1.0e9 + (br ? br[kk] : 0.0);"),
    ("causal_flipped", "valid[kk] = qi >= kk;", "valid[kk] = qi <= kk;"),
    ("len_off_by_one", "valid[kk] = kk < len;", "valid[kk] = kk <= len;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_backward_mutant(name, old, new, tmp_path):
    text = open(orc_mod._SRC_BWD).read()
    assert text.count(old) == 1, f"mutation site for {name} not found"
    src = os.path.join(tmp_path, f"{name}.c")
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    lib = orc_mod.load_library_bwd(orc.build(src, os.path.join(tmp_path, f"{name}.so")))
    bwd = functools.partial(orc.oracle_bwd, lib=lib)
    failed = False
    for kind in KINDS:
        try:
            _check_fd(_case(kind), bwd)
        except AssertionError:
            failed = True
            break
    assert failed, f"mutant {name} passed every finite-difference pin"


@pytest.mark.parametrize("kind", KINDS)
def test_query_row_subset_matches_full(kind):
    """Evaluating only some query rows gives exactly the full result's dQ and
    dBias on those rows (zero elsewhere): each row's gradient terms do not
    depend on the other rows."""
    c = _case(kind, N=3, Q=4, seed=11)
    if kind == "dense":
        c["mk"] = dict(mask=np.random.default_rng(2).random((1, 3, 5)) < 0.6)
    elif kind == "kv_lengths":
        c["mk"] = dict(kv_lengths=np.array([[3, 0, 5]], dtype=np.int32))
    args = (c["q"], c["k"], c["v"], c["bias"])
    full = orc.oracle_bwd(*args, dout=c["dout"], scale=c["scale"], **c["mk"])
    sel = [3, 0]
    part = orc.oracle_bwd(*args, dout=c["dout"], scale=c["scale"], q_rows=sel, **c["mk"])
    others = [q for q in range(4) if q not in sel]
    assert np.array_equal(part[0][:, :, :, sel], full[0][:, :, :, sel])
    assert not part[0][:, :, :, others].any()
    if c["bias"] is not None:
        assert np.array_equal(part[3][:, :, :, sel], full[3][:, :, :, sel])
        assert not part[3][:, :, :, others].any()
    with pytest.raises(RuntimeError):
        orc.oracle_bwd(*args, dout=c["dout"], scale=c["scale"], q_rows=[4], **c["mk"])
