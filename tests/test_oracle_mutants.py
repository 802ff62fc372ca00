"""Every planted mistake in the oracle is caught by at least one pin.

The oracle source carries six deliberate mistakes behind a compile-time
switch (decay dropped, decay on the value axis, transposed prediction,
wrong sign of the correction, taps reversed, output read before the update).
Each variant is built here, on the CPU, and run through the pins."""

import pytest

import oracle
import oracle_pins as P

MUTANTS = {1: "decay dropped", 2: "decay on value axis", 3: "S k instead of S^T k",
           4: "sign of correction", 5: "conv taps reversed", 6: "output before update"}


@pytest.mark.parametrize("m", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_mutant_is_caught(m, tmp_path):
    orc = oracle.load_mutant(m, tmp_path)
    assert orc.mutant == m
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {m} ({MUTANTS[m]}) passed every pin"
