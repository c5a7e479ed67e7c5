"""The oracle against its pins: printed worked examples, closed forms, brute
force on tiny inputs and invariants (no GPU)."""
import types

import pytest

import oracle.accounting
import oracle.alloc_model
import oracle.attention
import oracle.layout
import pins

REAL = types.SimpleNamespace(alloc_model=oracle.alloc_model, layout=oracle.layout,
                             attention=oracle.attention, accounting=oracle.accounting)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(REAL)
