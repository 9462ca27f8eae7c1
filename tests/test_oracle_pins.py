"""Runs every oracle pin (tests/oracle_pins.py) against the built oracle."""
import inspect

import pytest

import oracle
import oracle_pins

PINS = [(n, f) for n, f in inspect.getmembers(oracle_pins, inspect.isfunction)
        if n.startswith("pin_")]


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("name,pin", PINS, ids=[n for n, _ in PINS])
def test_pin(lib, name, pin):
    pin(lib)
