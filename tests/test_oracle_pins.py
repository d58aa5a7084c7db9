"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.spmm_ref)


def test_bf16_widening_known_patterns():
    """IEEE facts: bf16 0x3F80 = 1, 0xBF80 = -1, 0x4049 = 3.140625,
    0x3F81 = 1 + 2^-7, 0x0001 = 2^-133 (smallest subnormal), 0x7F7F = largest
    finite bf16, 0x8000 = -0."""
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x3F81, 0x0001, 0x7F7F, 0x8000],
                    dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, 1.0 + 2.0 ** -7, 2.0 ** -133,
            (2.0 - 2.0 ** -7) * 2.0 ** 127, -0.0]
    got = oracle.widen_bf16(bits)
    assert list(got) == want
    assert np.signbit(got[-1])


def test_oracle_rejects_bad_rows():
    rowptr = np.array([0, 1], dtype=np.int32)
    colind = np.array([0], dtype=np.int32)
    vals = np.ones(1, dtype=np.float32)
    B = np.ones((1, 2), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.spmm_ref(rowptr, colind, vals, B, 2, rows=np.array([1]))


def test_oracle_thread_count_independent():
    """The row loop is parallel over independent rows only: the result does
    not depend on how rows are split over threads (compare a full run with
    per-row sampled runs)."""
    rng = np.random.default_rng(5)
    rowptr, colind = oracle_pins.random_csr(rng, 64, 64, 0.3)
    vals = rng.standard_normal(colind.shape[0]).astype(np.float32)
    B = rng.standard_normal((64, 3)).astype(np.float32)
    C, _ = oracle.spmm_ref(rowptr, colind, vals, B, 3)
    for r in range(64):
        Cr, _ = oracle.spmm_ref(rowptr, colind, vals, B, 3, rows=[r])
        assert np.array_equal(Cr[0], C[r])
