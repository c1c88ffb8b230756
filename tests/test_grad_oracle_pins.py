import pytest

from tests import grad_pins


@pytest.mark.parametrize("pin", grad_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_grad_oracle_pin(pin):
    pin()
