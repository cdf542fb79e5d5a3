"""Planted mistakes in a copy of the oracle must be caught by the pins.

Each case copies ``oracle/moe_oracle.c`` to a temporary directory, changes one
expression into a plausible mistake (a dropped term, a wrong sign or index, an
unstable order, swapped halves), builds it with gcc and runs one of the pins of
``test_oracle_pins`` against that build.  The pin must fail.  Everything runs
on the CPU; the real oracle is never modified.
"""

import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")

MUTATIONS = [
    # name, original text, mistaken text, the pin that must catch it
    ("swapped_swiglu_halves", "act[i] = silu(h[i]) * h[I + i];",
     "act[i] = silu(h[I + i]) * h[i];", pins.test_forward_k1_unit_gate_is_dense_swiglu_ffn),
    ("sigmoid_sign", "return 1.0 / (1.0 + exp(-a));", "return 1.0 / (1.0 + exp(a));",
     pins.test_forward_scalar_closed_form),
    ("dropped_gate", "yt[c] += g * op[c];", "yt[c] += op[c];",
     lambda: pins.test_forward_matches_per_token_brute_force(*pins.FWD_CASES[0])),
    ("combine_wrong_slot", "const double *op = o + (int64_t)slot_pos[t * K + k] * H;",
     "const double *op = o + (int64_t)slot_pos[t * K] * H;",
     lambda: pins.test_forward_matches_per_token_brute_force(*pins.FWD_CASES[3])),
    ("unstable_scatter", "    for (int64_t s = 0; s < TK; ++s) {\n        int64_t e = load_id(ids, id_dt, s);\n        int32_t p = cursor[e]++;",
     "    for (int64_t s = TK - 1; s >= 0; --s) {\n        int64_t e = load_id(ids, id_dt, s);\n        int32_t p = cursor[e]++;",
     lambda: pins.test_route_matches_numpy(*pins.ROUTE_CASES[0])),
    ("offsets_off_by_one", "offsets[e + 1] = offsets[e] + counts[e];",
     "offsets[e + 1] = offsets[e] + counts[e] + (e == 0);", pins.test_route_hand_worked_fixture),
    ("swiglu_grad_sign", "dhp[i] = dact[i] * b * sg * (1.0 + a * (1.0 - sg));",
     "dhp[i] = dact[i] * b * sg * (1.0 - a * (1.0 - sg));", pins.test_backward_finite_differences),
    ("dW2_without_gate", "dOp[c] = g * dyr[c];", "dOp[c] = dyr[c];",
     pins.test_backward_linearity_identities),
    ("dx_transposed_index", "acc += dhp[j] * widen(W1, dt, row + j);",
     "acc += dhp[j] * widen(W1, dt, w1_base + (j % H) * 2 * I + (c % (2 * I)));",
     lambda: pins.test_backward_matches_autograd(*pins.FWD_CASES[3])),
    ("up_weight_wrong_expert", "const int64_t w1_base = e * H * 2 * I;\n    const int64_t w2_base",
     "const int64_t w1_base = ((e + 1) % 2) * H * 2 * I;\n    const int64_t w2_base",
     lambda: pins.test_forward_matches_per_token_brute_force(*pins.FWD_CASES[1])),
]


@pytest.mark.parametrize("name,old,new,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pin_catches_planted_mistake(tmp_path, name, old, new, pin):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "moe_oracle.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(lib),
                    str(mutated), "-lm"], check=True)
    oracle.use_library(str(lib))
    try:
        with pytest.raises((AssertionError, oracle.OracleError)):
            pin()
    finally:
        oracle.use_library(None)


def test_unmutated_pins_pass_through_variant_loader(tmp_path):
    lib = tmp_path / "libsame.so"
    shutil.copy(SRC, tmp_path / "moe_oracle.c")
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(lib),
                    str(tmp_path / "moe_oracle.c"), "-lm"], check=True)
    oracle.use_library(str(lib))
    try:
        pins.test_forward_k1_unit_gate_is_dense_swiglu_ffn()
        pins.test_backward_finite_differences()
    finally:
        oracle.use_library(None)
