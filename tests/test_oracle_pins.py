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


def test_down_wrapper_matches_forward():
    """oracle.down (one expert's down projection of one act row), weighted and
    summed over a token's slots, gives the layer output oracle.forward gives."""
    import numpy as np
    import synth
    spec = synth.small_spec(name="down-wrap", hidden=64, num_experts=5, top_k=2, expert_inter=96, seed=77)
    layer = synth.make_layer(spec)
    x = synth.make_tokens(spec, 6)
    o = oracle.forward(spec, layer, x, want_act=True)
    for t in range(6):
        y = sum(o["w"][t, j] * oracle.down(spec, layer, o["ids"][t, j], o["act"][t * 2 + j]) for j in range(2))
        assert np.allclose(y, o["y"][t], rtol=1e-12, atol=1e-12)
