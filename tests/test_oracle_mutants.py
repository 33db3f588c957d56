"""The oracle pins must catch plausible mistakes.

Each case copies oracle/gdn_oracle.c, plants one mistake in the copy (reading the
state before the update instead of after it, a flipped sign in the delta, a
dropped gate, a wrong query/key head, a transposed state row/column, a query or key
left unnormalised in the qk_norm variant), builds it
with gcc into a temporary directory, swaps it in for the real library for the
duration of the check, and requires that at least one pin fails.  Nothing on
the GPU is involved.
"""
import ctypes
import os
import subprocess

import pytest

from oracle import gdn_oracle as orc
from oracle import build as ob
import tests.test_oracle_pins as pins

MUTANTS = {
    "read_before_update": (
        "S[j] = a * S[j] + delta * kk[j];\n                oi += S[j] * qq[j];",
        "oi += S[j] * qq[j];\n                S[j] = a * S[j] + delta * kk[j];"),
    "delta_sign": ("const double delta = bt * (vi - a * u);", "const double delta = bt * (vi + a * u);"),
    "delta_missing_gate": ("const double delta = bt * (vi - a * u);", "const double delta = bt * (vi - u);"),
    "state_not_gated": ("S[j] = a * S[j] + delta * kk[j];", "S[j] = S[j] + delta * kk[j];"),
    "beta_dropped": ("const double delta = bt * (vi - a * u);", "const double delta = (vi - a * u);"),
    "wrong_head_map": ("const int hk = h / (Hv / Hk);\n    double *S", "const int hk = h % Hk;\n    double *S"),
    "state_transposed": ("J->state_in[(((size_t)b * Hv + h) * dv + i) * dk + j] : 0.0;",
                         "J->state_in[(((size_t)b * Hv + h) * dk + j) * dv + i] : 0.0;"),
    "qk_norm_skips_q": ("if (J->qk_norm) { l2_normalise(kk, dk); l2_normalise(qq, dk); }",
                        "if (J->qk_norm) { l2_normalise(kk, dk); }"),
    "qk_norm_skips_k": ("if (J->qk_norm) { l2_normalise(kk, dk); l2_normalise(qq, dk); }",
                        "if (J->qk_norm) { l2_normalise(qq, dk); }"),
    "qk_norm_without_sqrt": ("1.0 / sqrt(ss + GDN_ORACLE_NORM_EPS)", "1.0 / (ss + GDN_ORACLE_NORM_EPS)"),
    "value_from_wrong_head": ("J->v[(tok * Hv + h) * dv + i];\n            for (int j = 0; j < dk; ++j) { kk",
                              "J->v[(tok * Hv + (h ^ 1)) * dv + i];\n            for (int j = 0; j < dk; ++j) { kk"),
}

PINS = [pins.test_exact_golden_fixture, pins.test_p2_write_then_read_orthonormal_keys,
        lambda: pins.test_p1_rank1_matches_literal(0), pins.test_p3_beta_zero_pure_decay,
        pins.test_p4_unit_gate_zero_beta_is_readout, pins.test_p5_single_token_closed_form,
        pins.test_orthogonal_keys_reduce_to_gated_linear_attention,
        pins.test_state_equals_unrolled_product_form, pins.test_p7_affine_in_initial_state,
        pins.test_p10_shared_heads_equal_duplicated_heads,
        pins.test_p13_qknorm_write_then_read_raw_keys, pins.test_p13_qknorm_scale_invariance]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(ob.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-pthread", "-std=c99", str(path), "-o",
                    str(lib), "-lm"], check=True)
    mutant = ctypes.CDLL(str(lib))
    P = ctypes.c_void_p
    for fn in ("gdn_oracle_seq_f64", "gdn_oracle_seq_f64_qknorm", "gdn_oracle_seq_f32"):
        getattr(mutant, fn).argtypes = [P, P, P, P, P, P, P, ctypes.c_int, P, P] + [ctypes.c_int] * 8
        getattr(mutant, fn).restype = ctypes.c_int
    saved = orc._lib()
    orc._LIB = mutant
    failed = []
    try:
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                failed.append(getattr(pin, "__name__", "lambda"))
    finally:
        orc._LIB = saved
    assert failed, f"no pin caught mutant {name}"
