"""Oracle work order against its pin (no GPU)."""

import oracle
from tests import pins


def test_lpt_pin():
    pins.pin_lpt(oracle.lpt_work_order)
