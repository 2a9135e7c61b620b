"""The CPU oracle against its pins (no GPU)."""

import pytest

import pins
from oracle import reference as ref


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ref)


@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("pin", [pins.pin_brute_topk, pins.pin_split_merge_identity,
                                 pins.pin_retopk_invariants, pins.pin_retopk_brute],
                         ids=lambda f: f.__name__)
def test_pin_more_seeds(pin, seed):
    pin(ref, seed=seed)
