"""Each plausible mistake planted in a copy of the SDDMM/FusedMM oracle's C
source must fail at least one pin.  Copies are made by text substitution in
a temporary directory; the committed oracle is untouched."""
import os
import subprocess

import pytest

import oracle
import oracle_sddmm_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "sddmm_ref.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("dot_wrong_operand", "acc = acc + c * b;", "acc = acc + c * c;"),
    ("dot_wrong_sign", "acc = acc + c * b;", "acc = acc - c * b;"),
    ("dot_skips_first_column", "for (n = 0; n < N; ++n) {\n        double c",
     "for (n = 1; n < N; ++n) {\n        double c"),
    ("dot_drops_last_column", "for (n = 0; n < N; ++n) {\n        double c",
     "for (n = 0; n < N - 1; ++n) {\n        double c"),
    ("B_row_of_output_row", "load_elem(B, kind, j * N + n)", "load_elem(B, kind, i * N + n)"),
    ("C_row_of_column", "load_elem(C, kind, i * N + n)", "load_elem(C, kind, j * N + n)"),
    ("B_transposed", "load_elem(B, kind, j * N + n)", "load_elem(B, kind, n * N + j)"),
    ("sddmm_column_of_first_entry", "dot_entry(i, colind[p], N",
     "dot_entry(i, colind[rowptr[i]], N"),
    ("sddmm_output_slot", "int64_t o = base + (p - rowptr[i]);", "int64_t o = base;"),
    ("sddmm_drops_last_entry", "for (p = rowptr[i]; p < rowptr[i + 1]; ++p) {\n            double bound;",
     "for (p = rowptr[i]; p < rowptr[i + 1] - 1; ++p) {\n            double bound;"),
    ("fused_uses_B_for_D", "load_elem(D, kind, j * N + n)", "load_elem(B, kind, j * N + n)"),
    ("fused_weight_is_bound", "e[n] = e[n] + a * d;", "e[n] = e[n] + bound * d;"),
    ("fused_D_of_output_row", "load_elem(D, kind, j * N + n)", "load_elem(D, kind, i * N + n)"),
    ("fused_not_zeroed", "            e[n] = 0.0;", "            e[n] = 1.0;"),
    ("fused_column_of_first_entry", "int64_t j = colind[p];", "int64_t j = colind[rowptr[i]];"),
    ("bound_signed", "s = s + fabs(c) * fabs(b);", "s = s + c * b;"),
    ("bf16_shift", "((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    ("sample_offsets", "out_off[r] = total;", "out_off[r] = 0;"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor missing: {old!r}"
    c_path = tmp_path / f"{name}.c"
    so_path = tmp_path / f"lib{name}.so"
    c_path.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", "-w", "-o", str(so_path), str(c_path), "-lm"],
                   check=True)
    return oracle.load_sddmm_library(str(so_path))


def _run_pins(lib):
    def sd(*a, **kw):
        return oracle.sddmm_ref(*a, library=lib, **kw)

    def fu(*a, **kw):
        return oracle.fusedmm_ref(*a, library=lib, **kw)

    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(sd, fu)
        except AssertionError:
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    assert _run_pins(_build_mutant(tmp_path, name, old, new)), \
        f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    assert _run_pins(_build_mutant(tmp_path, "control", "int", "int")) == []
