"""The oracle against its pins (CPU only).  See oracle_pins.py for what each
pin compares with; none of them compares the oracle with itself."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(None)


import attention_pins as AP
import oracle.attention as OA


@pytest.mark.parametrize("pin", AP.ATTENTION_PINS, ids=lambda f: f.__name__)
def test_attention_oracle_pin(pin):
    pin(OA.attention)
