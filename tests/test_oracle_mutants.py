"""Each plausible mistake planted in a copy of the oracle's C source must
fail at least one pin.  The copies are made by text substitution into a
temporary directory and compiled there; the committed oracle is untouched."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "spmm_ref.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("drop_last_entry", "p < rowptr[i + 1]; ++p", "p < rowptr[i + 1] - 1; ++p"),
    ("skip_first_entry", "for (p = rowptr[i];", "for (p = rowptr[i] + 1;"),
    ("wrong_sign", "acc[n] = acc[n] + s * b;", "acc[n] = acc[n] - s * b;"),
    ("value_of_first_entry", "load_elem(vals, val_kind, p);",
     "load_elem(vals, val_kind, rowptr[i]);"),
    ("column_of_first_entry", "int64_t k = colind[p];",
     "int64_t k = colind[rowptr[i]];"),
    ("transposed_B", "const int64_t brow = k * N;", "const int64_t brow = k;"),
    ("row_index_shift", "one_row(i, N,", "one_row(i > 0 ? i - 1 : 0, N,"),
    ("acc_not_zeroed", "acc[n] = 0.0;", "acc[n] = 1.0;"),
    ("bound_signed", "fabs(s) * fabs(b)", "s * b"),
    ("bound_sum", "fabs(s) * fabs(b)", "fabs(s) + fabs(b)"),
    ("bf16_shift", "((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    ("bf16_low_half", "((uint32_t)bits) << 16", "((uint32_t)bits)"),
    ("float_rounding", "return (double)((const float *)base)[idx];",
     "return (double)(float)(0.5f * 2.0f * ((const float *)base)[idx] * 1.0000001f);"),
    ("sample_maps_to_position", "int64_t i = rows ? rows[r] : r;",
     "int64_t i = rows ? r % M : r;"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor missing: {old!r}"
    mutated = src.replace(old, new)
    c_path = tmp_path / f"{name}.c"
    so_path = tmp_path / f"lib{name}.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", "-w", "-o", str(so_path), str(c_path), "-lm"],
                   check=True)
    return oracle.load_library(str(so_path))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    lib = _build_mutant(tmp_path, name, old, new)

    def ref(*args, **kw):
        return oracle.spmm_ref(*args, library=lib, **kw)

    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(ref)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    """Control: a copy built the same way with no change passes all pins."""
    lib = _build_mutant(tmp_path, "control", "int", "int")

    def ref(*args, **kw):
        return oracle.spmm_ref(*args, library=lib, **kw)

    for pin in oracle_pins.ALL_PINS:
        pin(ref)
