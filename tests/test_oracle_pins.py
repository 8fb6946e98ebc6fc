"""The CPU oracle against its pins (hand-worked closed forms, binary16
conversions, float64 library routines, invariants).  CPU only."""
import pytest

import oracle
from pins import PINS, load_hand_cases, run_hand_case


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("case", load_hand_cases(), ids=lambda c: c["id"])
def test_hand_case(orc, case):
    run_hand_case(orc, case)


@pytest.mark.parametrize("pin", [p for p in PINS if p.__name__ != "pin_hand_cases"],
                         ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
