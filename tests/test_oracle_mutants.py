"""The oracle's pins must catch plausible mistakes.  Each case plants one
mistake in a copy of the oracle's C source (on the CPU, in a temp dir), loads
it in place of the real library and checks that at least one pin fails."""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "tgref.c")

MUTANTS = {
    "dropped_last_term": ("for (int64_t k = 0; k < K; k++)\n        s += arow[k] * bcol[k];",
                          "for (int64_t k = 0; k + 1 < K; k++)\n        s += arow[k] * bcol[k];"),
    "wrong_sign": ("s += arow[k] * bcol[k];", "s -= arow[k] * bcol[k];"),
    "bias_wrong_index": ("s = s + (double)bias[j];", "s = s + (double)bias[0];"),
    "no_relu": ("s = (s > 0.0) ? s : 0.0;", "s = s;"),
    "relu_inverted": ("s = (s > 0.0) ? s : 0.0;", "s = (s < 0.0) ? s : 0.0;"),
    "columns_of_B_swapped": ("bt[j * K + k] = tgref_f16_decode(elem_b(B, op_b, ldb, k, j));",
                             "bt[j * K + k] = tgref_f16_decode(elem_b(B, op_b, ldb, k, N - 1 - j));"),
    "lda_ignored": ("a[i * K + k] = tgref_f16_decode(elem_a(A, op_a, lda, i, k));",
                    "a[i * K + k] = tgref_f16_decode(elem_a(A, op_a, K, i, k));"),
    "transposed_a_not_transposed": ("return op_a ? A[k * lda + i] : A[i * lda + k];",
                                    "return op_a ? A[i * lda + k] : A[i * lda + k];"),
    "transposed_b_ignores_ldb": (
        "bt[j * K + k] = tgref_f16_decode(elem_b(B, op_b, ldb, k, j));",
        "bt[j * K + k] = tgref_f16_decode(elem_b(B, op_b, op_b ? K : ldb, k, j));"),
    "round_half_up": ("double n = rint(a / q);", "double n = floor(a / q + 0.5);"),
    "subnormal_scale": ("v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    "float_accumulator": ("double s = 0.0;\n    for (int64_t k = 0; k < K; k++)",
                          "float s = 0.0f;\n    for (int64_t k = 0; k < K; k++)"),
}


def _pin_suite():
    yield pins.test_decode_all_patterns_match_numpy
    yield pins.test_encode_midpoints_and_neighbours_match_numpy
    yield lambda: pins.test_identity_B_gives_A(37, 45)
    yield lambda: pins.test_fused_with_zero_A_is_relu_of_bias()
    yield lambda: pins.test_K0_gives_zero_or_relu_bias()
    yield pins.test_padded_leading_dimensions_ignore_padding
    yield pins.test_integer_inputs_are_exact_at_large_K
    yield pins.test_transposed_operands_match_numpy_transposes
    yield lambda: pins.test_transposed_brute_force_exact(5, 3, 7, 1, 1)
    for M, N, K in [(7, 5, 3), (4, 4, 4)]:
        for kind in ("uniform", "normal_scaled"):
            for fused in (False, True):
                yield (lambda M=M, N=N, K=K, kind=kind, fused=fused:
                       pins.test_brute_force_exact(M, N, K, kind, fused))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site not found: " + name
    mutated = src.replace(old, new)
    c = tmp_path / "tgref_mut.c"
    so = tmp_path / "libtgref_mut.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
                    "-ffp-contract=off", "-o", str(so), str(c), "-lm"], check=True)
    real = oracle.lib()
    mut = ctypes.CDLL(str(so))
    for fn in ("tgref_f16_decode", "tgref_f16_encode", "tgref_decode_array", "tgref_to_f32",
               "tgref_to_f16", "tgref_gemm", "tgref_gemm_entries", "tgref_gemm_ex",
               "tgref_gemm_entries_ex"):
        getattr(mut, fn).argtypes = getattr(real, fn).argtypes
        getattr(mut, fn).restype = getattr(real, fn).restype
    caught = []
    oracle._lib = mut
    try:
        for pin in _pin_suite():
            try:
                pin()
            except AssertionError:
                caught.append(pin)
                break
    finally:
        oracle._lib = real
    assert caught, "no pin caught the planted mistake " + name
