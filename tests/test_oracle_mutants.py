"""The pins must reject plausible mistakes in the oracle.

Each mutant is a copy of triattn_oracle.c with one deliberate error (a dropped
or misplaced term, a wrong sign, index or operand), compiled on the CPU into a
temporary library.  Running the pin checks of tests/oracle_pins.py against it
must fail at least one of them.  Only the oracle is mutated; nothing here
touches a GPU.
"""
import functools
import os
import shutil

import pytest

import oracle as orc
from oracle import oracle as orc_mod
from tests import oracle_pins as pins

SRC = orc_mod._SRC

# (name, original text, replacement)
MUTANTS = [
    ("drop_bias", "a->scale * dot + (brow ? brow[kk] : 0.0)", "a->scale * dot"),
    ("bias_before_scale", "a->scale * dot + (brow ? brow[kk] : 0.0)",
     "a->scale * (dot + (brow ? brow[kk] : 0.0))"),
    ("bias_sign", "a->scale * dot + (brow ? brow[kk] : 0.0)",
     "a->scale * dot - (brow ? brow[kk] : 0.0)"),
    ("bias_q_index", "((b * H + h) * Q + qi) * K", "((b * H + h) * Q + (Q - 1 - qi)) * K"),
    ("bias_h_index", "((b * H + h) * Q + qi) * K", "((b * H + (H - 1 - h)) * Q + qi) * K"),
    ("bias_per_n", "((b * H + h) * Q + qi) * K", "((b * H + h) * Q + qi) * K + (n % 2)"),
    ("default_scale_1_over_d", "1.0 / sqrt((double)D)", "1.0 / (double)D"),
    ("masked_additive", "z[kk] = MASKED_LOGIT;",
     "z[kk] = MASKED_LOGIT + (brow ? brow[kk] : 0.0);"),
    ("masked_zero", "z[kk] = MASKED_LOGIT;", "z[kk] = 0.0;"),
    ("dense_ignored", "valid = a->dense[(b * N + n) * K + kk] != 0;", "valid = 1;"),
    ("dense_inverted", "valid = a->dense[(b * N + n) * K + kk] != 0;",
     "valid = a->dense[(b * N + n) * K + kk] == 0;"),
    ("dense_n_index", "valid = a->dense[(b * N + n) * K + kk] != 0;",
     "valid = a->dense[(b * N + (N - 1 - n)) * K + kk] != 0;"),
    ("len_off_by_one", "valid = kk < valid_len;", "valid = kk <= valid_len;"),
    ("causal_direction", "(qi >= kk)", "(qi <= kk)"),
    ("causal_strict", "(qi >= kk)", "(qi > kk)"),
    ("full_not_visited", "if (full[j]) listed[j] = 1;", "(void)0;"),
    ("mod_on_full_blocks", "} else if (!full[blk]) {", "} else {"),
    ("block_row_uses_kv_block", "qi / a->q_block", "qi / a->kv_block"),
    ("instance_stride_h", "h * a->stride_h", "h * a->stride_n"),
    ("reads_past_count", "for (int64_t j = 0; j < count; ++j)",
     "for (int64_t j = 0; j < width; ++j)"),
    ("lse_log2", "a->lse[pos] = m + log(l);", "a->lse[pos] = m + log2(l);"),
    ("lse_without_max", "a->lse[pos] = m + log(l);", "a->lse[pos] = log(l);"),
    ("max_is_lse", "a->mx[pos] = m;", "a->mx[pos] = m + log(l);"),
    ("no_normalisation", "orow[d] = acc / l;", "orow[d] = acc;"),
    ("v_d_reversed", "vbase[kk * D + d]", "vbase[kk * D + (D - 1 - d)]"),
    ("k_is_v", "const double *kbase = a->k + bnh * K * D;",
     "const double *kbase = a->v + bnh * K * D;"),
    ("dot_drops_last_d", "for (int64_t d = 0; d < D; ++d) dot += qrow[d] * krow[d];",
     "for (int64_t d = 0; d + 1 < D; ++d) dot += qrow[d] * krow[d];"),
    ("q_row_zero", "const double *qrow = a->q + row * D;",
     "const double *qrow = a->q + (row - qi) * D;"),
    ("max_from_first_key", "if (z[kk] > m) m = z[kk];", "(void)0;"),
]


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new, mutant_dir):
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    src = os.path.join(mutant_dir, f"{name}.c")
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    lib = orc.load_library(orc.build(src, os.path.join(mutant_dir, f"{name}.so")))
    fwd = functools.partial(orc.oracle_fwd, lib=lib)
    failed = []
    for check_name, check in pins.ALL_CHECKS:
        try:
            check(fwd)
        except AssertionError:
            failed.append(check_name)
        except RuntimeError:
            failed.append(check_name + "(error)")
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(mutant_dir):
    src = os.path.join(mutant_dir, "clean.c")
    shutil.copy(SRC, src)
    lib = orc.load_library(orc.build(src, os.path.join(mutant_dir, "clean.so")))
    fwd = functools.partial(orc.oracle_fwd, lib=lib)
    for _, check in pins.ALL_CHECKS:
        check(fwd)
