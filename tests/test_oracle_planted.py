"""Plants plausible mistakes in a COPY of the oracle's C source, on the CPU, and
checks that the pins reject every one of them.  This is what makes the pins
worth trusting: a dropped term, a flipped sign, a wrong index, a wrong scale or
an off-by-one window each fails at least one of them."""
import math
import os
import shutil

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "atf_oracle.c")


def _checks(o):
    """Each pin, called on the candidate oracle; returns the names that fail."""
    cases = {
        "closed_forms": lambda: pins.test_window_closed_forms(o),
        "structure": lambda: pins.test_window_structure(o, 64, 1e4, 1.0),
        "count": lambda: pins.test_count_closed_form_equals_brute_force(o, 200, 16, 10.0, 1.0),
        "enumerated": lambda: pins.test_oracle_enumerated_count_matches(o, True),
        "alpha_inf": lambda: pins.test_alpha_inf_equals_dense(o, True),
        "alpha_inf_nc": lambda: pins.test_alpha_inf_equals_dense(o, False),
        "decode_dense": lambda: pins.test_alpha_inf_decode_equals_dense(o),
        "single_pair": lambda: [pins.test_single_pair_explicit_logits(o, p, True) for p in (0, 7, 15)],
        "single_pair_nc": lambda: pins.test_single_pair_explicit_logits(o, 7, False),
        "gqa": lambda: pins.test_gqa_equals_repeated_heads(o),
        "reachable": lambda: pins.test_every_causal_key_reachable(o),
        "slowest": lambda: pins.test_slowest_pair_only_equals_dense(o, 1.0),
        "gptj_dense": lambda: pins.test_gptj_alpha_inf_equals_dense(o, True),
        "gptj_moved": lambda: pins.test_gptj_equals_halfsplit_on_moved_dims(o, 1.0),
    }
    failed = []
    for name, fn in cases.items():
        try:
            fn()
        except (AssertionError, ValueError):
            failed.append(name)
    return failed


MUTATIONS = {
    "rotation_sign": ("y[il] = lo * c - hi * s;", "y[il] = lo * c + hi * s;"),
    "dropped_hi_term": ("double term = qrot[il] * kr[il] + qrot[ih] * kr[ih];",
                        "double term = qrot[il] * kr[il];"),
    "gptj_dims_swapped": ("{ return layout ? 2 * p : p; }\nstatic int orc_dim_hi(int p, int P, int layout) "
                          "{ return layout ? 2 * p + 1 : p + P; }",
                          "{ return layout ? 2 * p + 1 : p; }\nstatic int orc_dim_hi(int p, int P, int layout) "
                          "{ return layout ? 2 * p : p + P; }"),
    "gptj_layout_ignored_lo": ("static int orc_dim_lo(int p, int P, int layout) { return layout ? 2 * p : p; }",
                               "static int orc_dim_lo(int p, int P, int layout) { return p; }"),
    "window_exclusive": ("return Wp == ORC_W_INF || dist <= Wp;", "return Wp == ORC_W_INF || dist < Wp;"),
    "window_floor": ("double w = ceil(alpha * lambda);", "double w = floor(alpha * lambda);"),
    "last_pair_cut": ("if (p == P - 1 || isinf(alpha)) {", "if (isinf(alpha)) {"),
    "scale_1_over_d": ("logit[j] = s / sqrt((double)d);", "logit[j] = s / (double)d;"),
    "theta_exponent": ("theta[p] = pow(base, -2.0 * (double)p / (double)d);",
                       "theta[p] = pow(base, -1.0 * (double)p / (double)d);"),
    "causal_flip": ("if (causal && delta < 0) {", "if (causal && delta > 0) {"),
    "gqa_modulo": ("if (rows[3 * r] != b || rows[3 * r + 1] / group != hk)",
                   "if (rows[3 * r] != b || rows[3 * r + 1] % Hkv != hk)"),
    "value_row_of_query": ("const float *vr = vh + (size_t)j * d;",
                           "const float *vr = vh + (size_t)(j < i ? j + 1 : j) * d;"),
    "dropped_to_minus_inf": ("                                skipped_here += 1;",
                             "                                skipped_here += 1; s = -INFINITY;"),
    "closed_form_off_by_one": ("int64_t n = S - 1 - W[p];", "int64_t n = S - W[p];"),
}


def test_unmutated_copy_passes(tmp_path):
    src = tmp_path / "atf_oracle.c"
    shutil.copy(SRC, src)
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / "lib.so"))
    assert _checks(oracle.Oracle(lib)) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor not found: " + name
    src = tmp_path / "atf_oracle.c"
    src.write_text(text.replace(old, new, 1))
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / "lib.so"))
    failed = _checks(oracle.Oracle(lib))
    assert failed, "planted mistake %r passed every pin" % name
