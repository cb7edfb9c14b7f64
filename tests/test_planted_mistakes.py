"""Each deliberate mistake compiled into the oracle (OR_PLANT=n) must be caught
by at least one pin, and the clean build must pass them all. Mistakes are
planted in the oracle only, on the CPU."""
import os

import pytest

import oracle
from tests import oracle_pins

PLANTS = {
    1: "zero point dropped",
    2: "sign of (q - z) flipped",
    3: "neighbouring groups share a scale",
    4: "activations read transposed",
    5: "nibble order reversed",
    6: "fp16 rounding truncates",
    7: "fp16 subnormals decoded with a hidden bit",
}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p].replace(" ", "_"))
def test_plant_is_caught(tmp_path, plant):
    path = oracle.build(out_path=os.path.join(tmp_path, f"liboracle_plant{plant}.so"), plant=plant)
    o = oracle.Oracle(path)
    assert o.plant == plant
    caught = []
    for pin in oracle_pins.PINS:
        try:
            pin(o)
        except (AssertionError, ValueError) as e:  # noqa: PERF203
            caught.append(pin.__name__)
    assert caught, f"no pin caught planted mistake {plant}: {PLANTS[plant]}"
