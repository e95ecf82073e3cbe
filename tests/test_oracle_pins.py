"""The CPU oracle against its pins, and the pins against planted mistakes."""
import pytest

import oracle
import pins


@pytest.fixture(autouse=True)
def _clean_oracle():
    oracle.set_mutant(0)
    yield
    oracle.set_mutant(0)


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


@pytest.mark.parametrize("mutant", sorted(oracle.MUTANTS), ids=lambda m: oracle.MUTANTS[m])
def test_planted_mistake_fails_a_pin(mutant):
    oracle.set_mutant(mutant)
    caught = []
    for pin in pins.PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    oracle.set_mutant(0)
    assert caught, f"no pin catches the planted mistake: {oracle.MUTANTS[mutant]}"
