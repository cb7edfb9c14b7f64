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
    8: "symmetric quantizer scale absmax / 8",
    9: "asymmetric quantizer drops the zero point",
    10: "activation code scale absmax / 128",
    11: "activation scale of row 0 used for every row",
    12: "integer-sum product drops the zero point",
    13: "scale and zero rows reversed past the first row tile",
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


# Mistakes in the SwiGLU composition (the Python part of the oracle).
def _swap_gate_up(real):
    def mutant(o, qg, sg, zg, qu, su, zu, x):
        return real(o, qu, su, zu, qg, sg, zg, x)
    return mutant


def _sigmoid_for_silu(real_silu):
    def mutant(v):
        v = oracle.np.asarray(v, dtype=oracle.np.float64)
        return 1.0 / (1.0 + oracle.np.exp(-v))
    return mutant


def _silu_sign_flipped(real_silu):
    def mutant(v):
        v = oracle.np.asarray(v, dtype=oracle.np.float64)
        return v / (1.0 + oracle.np.exp(v))
    return mutant


SWIGLU_PLANTS = {
    "gate_and_up_swapped": ("gemv_swiglu", _swap_gate_up),
    "sigmoid_instead_of_silu": ("silu", _sigmoid_for_silu),
    "silu_exponent_sign_flipped": ("silu", _silu_sign_flipped),
}


@pytest.mark.parametrize("name", sorted(SWIGLU_PLANTS))
def test_swiglu_plant_is_caught(monkeypatch, name):
    attr, make = SWIGLU_PLANTS[name]
    monkeypatch.setattr(oracle, attr, make(getattr(oracle, attr)))
    o = oracle.get()
    caught = []
    for pin in oracle_pins.PINS:
        if "silu" not in pin.__name__ and "swiglu" not in pin.__name__:
            continue
        try:
            pin(o)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught planted SwiGLU mistake {name}"
