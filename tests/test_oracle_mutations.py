"""Each planted mistake in the oracle must make at least one pin fail
("run the arm without the change and watch it fail"). Mistakes are planted on
the CPU, in the oracle only, through its test-only mutation switch."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("name", sorted(oracle.MUTATIONS))
def test_mutation_is_caught(oracle_lib, name):
    failed = []
    with oracle.mutation(name):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"


def test_pins_pass_without_mutation(oracle_lib):
    for pin in oracle_pins.ALL_PINS:
        pin()
