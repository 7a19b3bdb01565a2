"""The oracle's pins are strong enough to catch plausible slips (no GPU).

Each mutant is a copy of oracle/bha_oracle.c with one deliberate mistake of
the kind a reimplementation of the pages' formulas could make, built with gcc
into a temporary directory and swapped in for the real oracle. The pins of
test_oracle.py are then run against it: every mutant must fail at least one,
and the unmodified source, built the same way, must pass them all (so the
harness itself is sound). Nothing here touches the real oracle library.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle as T

SRC = os.path.join(os.path.dirname(oracle.__file__), "bha_oracle.c")

# (name, text in bha_oracle.c, replacement): each text occurs exactly once
MUTANTS = [
    ("row maximum with the wrong sign in the gate factor",
     "const double g = gamma * exp(-m);", "const double g = gamma * exp(m);"),
    ("linear term dropped from the denominator", "den += g * lin_den;", "den += 0.0 * lin_den;"),
    ("second half of phi without the minus sign",
     "phi[fw + j] = exp(-u[j] - mn);", "phi[fw + j] = exp(u[j] - mn);"),
    ("W read transposed", "acc += x[c] * w[(size_t)j * d + c];", "acc += x[c] * w[(size_t)c * fw + j];"),
    ("commit folds phi(k) k^T instead of phi(k) v^T",
     "S[(size_t)f * d + c] += ph[f] * v[(size_t)t * d + c];",
     "S[(size_t)f * d + c] += ph[f] * k[(size_t)t * d + c];"),
    ("softmax scale 1/d instead of 1/sqrt(d)",
     "const double c = (scale > 0.0) ? scale : 1.0 / sqrt((double)d);\n    double* s = (double*)malloc(sizeof(double) * (size_t)B);",
     "const double c = (scale > 0.0) ? scale : 1.0 / (double)d;\n    double* s = (double*)malloc(sizeof(double) * (size_t)B);"),
    ("causal mask inside the block", "            s[j] = c * acc;\n        }\n        double m = s[0];\n        for (int j = 1; j < B; ++j)",
     "            s[j] = j > i ? -1e300 : c * acc;\n        }\n        double m = s[0];\n        for (int j = 1; j < B; ++j)"),
    ("phi of the key instead of the query in the linear read",
     "bha_ref_phi(qi, w, d, fw, ph);", "bha_ref_phi(k + (size_t)i * d, w, d, fw, ph);"),
    ("every head uses head 0's map in the batched driver",
     "const double* wh = jb->w + (size_t)h * jb->fw * jb->d;", "const double* wh = jb->w;"),
    ("normaliser Z counts features instead of phi", "Z[f] += ph[f];", "Z[f] += 1.0;"),
    ("first half of phi not normalised", "for (int j = 0; j < fw; ++j) phi[j] /= sum;", ""),
    ("linear read ignores phi in the denominator", "lin_den += ph[f] * Z[f];", "lin_den += Z[f];"),
    ("softmax denominator without the row maximum", "for (int j = 0; j < B; ++j) den += exp(s[j] - m);",
     "for (int j = 0; j < B; ++j) den += exp(s[j]);"),
    ("prefix attention skips the block's own keys", "const int nk = np + B;", "const int nk = np + (B > 1 ? B - 1 : B);"),
]

# the pins run against each mutant: (test function, arguments)
PINS = [
    (T.test_phi_halves_positive_and_normalised, (6, 3, 5)),
    (T.test_phi_negated_input_swaps_halves, (6, 3, 5)),
    (T.test_phi_zero_matrix_is_uniform, ()),
    (T.test_phi_two_column_closed_form, ()),
    (T.test_phi_matches_library_softmax, (6, 3, 5)),
    (T.test_normaliser_halves_count_tokens, (6, 3, 5)),
    (T.test_incremental_commits_equal_one_shot_build, (6, 3, 5)),
    (T.test_single_token_state_reads_back_its_value, (6, 3, 5)),
    (T.test_state_read_equals_bruteforce_over_prior_tokens, (6, 3, 5)),
    (T.test_gate_zero_is_block_softmax_attention, (6, 3, 5)),
    (T.test_empty_state_is_block_softmax_attention, (6, 3, 5)),
    (T.test_explicit_softmax_scale_is_used, ()),
    (T.test_forward_equals_bruteforce_over_prefix, (6, 3, 5, 3.0)),
    (T.test_constant_values_give_constant_output, ()),
    (T.test_output_in_convex_hull_of_values, ()),
    (T.test_large_gate_limit_is_normalised_linear_attention, ()),
    (T.test_zero_matrix_closed_form, ()),
    (T.test_state_and_gate_rescaling_invariance, ()),
    (T.test_single_token_block_closed_form, ()),
    (T.test_batched_forward_matches_pairs, ()),
    (T.test_batched_commit_matches_pairs, ()),
    (T.test_prefix_attention_is_softmax_attention_over_prefix_and_block, (8, 4, 13)),
    (T.test_prefix_attention_explicit_scale_and_constant_values, ()),
]


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-ffp-contract=off", str(src),
                    "-o", str(lib), "-lm"], check=True)
    return oracle._open(str(lib))


def _failed_pins(monkeypatch, lib):
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = []
    for fn, args in PINS:
        try:
            fn(*args)
        except AssertionError:
            failed.append(fn.__name__)
    return failed


def test_unmodified_source_passes_every_pin(tmp_path, monkeypatch):
    with open(SRC) as f:
        text = f.read()
    assert _failed_pins(monkeypatch, _build(tmp_path, "original", text)) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(tmp_path, monkeypatch, name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    failed = _failed_pins(monkeypatch, _build(tmp_path, "mutant", text.replace(old, new)))
    print(f"mutant '{name}': fails {len(failed)} of {len(PINS)} pins ({', '.join(failed[:4])}"
          f"{', ...' if len(failed) > 4 else ''})")
    assert failed, f"no pin catches the mutant '{name}'"
