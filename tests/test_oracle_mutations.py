"""The oracle pins must reject plausible mistakes.

Each case compiles a copy of cce_oracle.c with one planted mistake (on the CPU,
into a temporary directory), swaps it in for the real oracle, and checks that
at least one pin of test_oracle.py fails.  The real oracle is restored after.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "cce_oracle.c")

MUTANTS = {
    "code order reversed in the word": ("(bits * (d % per_word))", "(bits * (per_word - 1 - d % per_word))"),
    "group index from the wrong axis": ("gi = v * groups_per_row + d / group", "gi = v * groups_per_row + d % groups_per_row"),
    "bias dropped": ("(double)q + (double)biases[gi]", "(double)q"),
    "softcap derivative missing": ("dc = 1.0 - th * th;", "dc = 1.0;"),
    "softmax term with the wrong sign": ("(onehot - exp(y[v] - l))", "(onehot + exp(y[v] - l))"),
    "normalizer without the max shift": ("const double l = mx + log(se);", "const double l = log(se);"),
    "out-of-range target takes row 0": ("(tgt_in ? y[tg] : 0.0)", "(tgt_in ? y[tg] : y[0])"),
    "cotangent ignored": ("const double gt = g ? g[t] : 1.0;", "const double gt = 1.0;"),
    "hidden state read transposed": ("h[t * H + d]", "h[d * M + t]"),
    "mask ignored": ("if (mask && mask[t] == 0) {", "if (0) {"),
    "softcap applied as plain scaling": ("softcap * tanh(z[v] / softcap)", "z[v] / softcap"),
}

BATTERY = [
    (pins.test_code_order_and_group_index_from_hex_words, dict(bits=4)),
    (pins.test_code_order_and_group_index_from_hex_words, dict(bits=8)),
    (pins.test_identical_rows_give_uniform_softmax, dict(softcap=5.0)),
    (pins.test_two_way_closed_form, dict(softcap=0.0)),
    (pins.test_two_way_closed_form, dict(softcap=3.0)),
    (pins.test_probabilities_sum_to_one_and_lse_bounds, dict(softcap=2.0)),
    (pins.test_gradient_matches_central_differences, dict(bits=8, softcap=4.0, target=3)),
    (pins.test_gradient_matches_central_differences, dict(bits=4, softcap=4.0, target=-1)),
    (pins.test_linearity_in_g_and_large_cap, {}),
    (pins.test_mask_zeroes_exactly_and_isolates, {}),
    (pins.test_against_torch_float64_autograd, dict(bits=8, softcap=30.0)),
]


def _battery_passes() -> bool:
    for fn, kw in BATTERY:
        try:
            fn(**kw)
        except AssertionError:
            return False
    return True


def test_real_oracle_passes_battery():
    assert _battery_passes()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished: " + name
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(path), "-lm"])
    saved = oracle._lib
    oracle._lib = oracle.load(str(so))
    try:
        caught = not _battery_passes()
    finally:
        oracle._lib = saved
    assert caught, "no pin rejects: " + name
