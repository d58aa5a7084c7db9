"""The SDDMM and FusedMM oracles against their pins (see oracle_sddmm_pins)."""
import pytest

import oracle
import oracle_sddmm_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_pin(pin):
    pin(oracle.sddmm_ref, oracle.fusedmm_ref)
