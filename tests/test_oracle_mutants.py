"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake in a temporary copy of the oracle's C source
(a flipped erase sign, a decayed write, a missing scale, a transposed state
layout, ...), builds it, and runs the pins of ``test_oracle_pins`` against
it: at least one pin has to fail.  The committed oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle
from oracle.build import SRC
import test_oracle_pins as pins
import test_oracle_pins_decay as dpins

PINS = [
    pins.test_hand_worked_example,
    pins.test_p1_identity_when_no_write_and_no_decay,
    pins.test_p2_pure_decay,
    pins.test_p3_zero_gate_resets_to_rank_one,
    pins.test_p4_orthonormal_keys_exact_retrieval_and_overwrite,
    pins.test_p5_single_token_from_zero_state,
    pins.test_p11_householder_reflection_preserves_norm,
    lambda o: pins.test_p9_brute_force_product_form(o, 20, 1, 6, 2, 4, 4, True),
    lambda o: pins.test_p9_brute_force_product_form(o, 22, 1, 7, 3, 4, 2, True),
    pins.test_p9_brute_force_literal_gates_and_large_beta,
    pins.test_p10_contraction_bound,
]

# (name, original text, planted mistake)
MUTANTS = [
    ("erase_sign", "srow[j] - bt * w * kj", "srow[j] + bt * w * kj"),
    ("write_decayed", "a * (srow[j] - bt * w * kj) + bt * vi * kj", "a * (srow[j] - bt * w * kj + bt * vi * kj)"),
    ("write_without_beta", "+ bt * vi * kj", "+ vi * kj"),
    ("erase_without_beta", "srow[j] - bt * w * kj", "srow[j] - w * kj"),
    ("gate_linearised", "exp(orc_load(g, gb_dtype, bth))", "(1.0 + orc_load(g, gb_dtype, bth))"),
    ("missing_scale", "o[bth * dv + i] = acc * scale;", "o[bth * dv + i] = acc;"),
    ("scale_by_dv", "1.0 / sqrt((double)dk)", "1.0 / sqrt((double)dv)"),
    ("erase_probe_uses_q", "w += srow[j] * orc_load(k, qkv_dtype, bth * dk + j);",
     "w += srow[j] * orc_load(q, qkv_dtype, bth * dk + j);"),
    ("readout_with_k", "acc += srow[j] * orc_load(q, qkv_dtype, bth * dk + j);",
     "acc += srow[j] * orc_load(k, qkv_dtype, bth * dk + j);"),
    ("state_value_major", "s_out[((b * H + h) * dk + j) * dv + i]", "s_out[((b * H + h) * dv + i) * dk + j]"),
]


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant_dir, name, orig, bad):
    with open(SRC) as f:
        src = f.read()
    assert src.count(orig) >= 1, f"mutation site for {name} not found"
    src = src.replace(orig, bad)
    csrc = os.path.join(mutant_dir, f"{name}.c")
    lib = os.path.join(mutant_dir, f"lib{name}.so")
    with open(csrc, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", lib, csrc, "-lm"],
                   check=True)
    mutant = oracle.Oracle(lib)
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(getattr(pin, "__name__", "lambda"))
    assert failed, f"no pin detects the planted mistake {name!r}"


# the second rule (no erase), caught by its own pins
PINS_DECAY = [
    dpins.test_decay_hand_worked_example,
    lambda o: dpins.test_decay_matches_explicit_decayed_sums(o, 1, 1, 9, 2, 4, 3, "primary"),
    dpins.test_decay_pure_decay_and_single_token,
    dpins.test_decay_accumulates_where_the_delta_rule_overwrites,
]
MUTANTS_DECAY = [
    ("decay_write_decayed", "srow[j] = a * srow[j] + bt * vi * orc_load(k, qkv_dtype, bth * dk + j);",
     "srow[j] = a * (srow[j] + bt * vi * orc_load(k, qkv_dtype, bth * dk + j));"),
    ("decay_write_without_beta", "a * srow[j] + bt * vi * orc_load(", "a * srow[j] + vi * orc_load("),
    ("decay_not_applied", "srow[j] = a * srow[j] + bt", "srow[j] = srow[j] + bt"),
    ("decay_rule_erases", "if (rule == ORC_RULE_GATED_DECAY) {", "if (0) {"),
]


@pytest.mark.parametrize("name,orig,bad", MUTANTS_DECAY, ids=[m[0] for m in MUTANTS_DECAY])
def test_decay_pins_catch_planted_mistake(mutant_dir, name, orig, bad):
    with open(SRC) as f:
        src = f.read()
    assert src.count(orig) == 1, f"mutation site for {name} not unique"
    src = src.replace(orig, bad)
    csrc = os.path.join(mutant_dir, f"{name}.c")
    lib = os.path.join(mutant_dir, f"lib{name}.so")
    with open(csrc, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", lib, csrc, "-lm"],
                   check=True)
    mutant = oracle.Oracle(lib)
    failed = []
    for pin in PINS_DECAY:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(getattr(pin, "__name__", "lambda"))
    assert failed, f"no decay pin detects the planted mistake {name!r}"
