"""The CPU oracle against the pages' printed values, textbook routines and
closed forms (see ``oracle_checks.py`` for what each pin compares with)."""

import pytest

import oracle
import oracle_checks


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("check", oracle_checks.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(lib, check):
    check(lib)
