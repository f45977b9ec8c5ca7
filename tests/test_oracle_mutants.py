"""The pins have teeth: plausible mistakes planted in a copy of the oracle
(on the CPU, in a temporary directory) must each fail at least one pin.

Every mutation is a textual edit of oracle.c that compiles and stays in
bounds; the in-tree oracle is never modified.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    # assignment: tie rule, dropped term, wrong sign, wrong batch index, second-best
    "ties_to_highest_index": ("if (dist < best) {", "if (dist <= best) {"),
    "sign_flip_in_distance": ("const double diff = x[j] - c[j];",
                              "const double diff = x[j] + c[j];"),
    "dropped_last_dimension": ("for (int64_t j = 0; j < d; ++j) {\n                    const double diff",
                               "for (int64_t j = 0; j + 1 < d; ++j) {\n                    const double diff"),
    "centroids_of_problem_zero": ("const double* c = Cd + (b * K + k) * d;",
                                  "const double* c = Cd + k * d;"),
    "no_second_best": ("} else if (dist < second) {", "} else if (0) {"),
    "abs_instead_of_square": ("dist += diff * diff;\n                }\n                if (dist < best)",
                              "dist += fabs(diff);\n                }\n                if (dist < best)"),
    # update: divisor, empty rule, batch index of labels
    "mean_divisor_off_by_one": ("sums[k * d + j] / (double)cnt[k]",
                                "sums[k * d + j] / (double)(cnt[k] + 1)"),
    "empty_cluster_zeroed": (": decode_one(dtype_c, C_prev, o);", ": 0.0;"),
    "labels_of_problem_zero": ("const int32_t a = labels[b * N + i];",
                               "const int32_t a = labels[i];"),
    # decoding / encoding
    "f16_exponent_bias": ("mag = ldexp((double)((1u << fbits) + f), (int)e - bias - fbits);",
                          "mag = ldexp((double)((1u << fbits) + f), (int)e - bias - fbits + (ebits == 5));"),
    "truncating_encoder": ("double r = ldexp(rint(ldexp(v, -qexp)), qexp);",
                           "double r = ldexp(floor(ldexp(v, -qexp)), qexp);"),
    "no_subnormal_decode": ("mag = ldexp((double)f, 1 - bias - fbits);", "mag = 0.0;"),
}


@pytest.fixture(scope="module")
def source():
    with open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(source.replace(old, new))
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / f"liboracle_{name}.so"))
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
