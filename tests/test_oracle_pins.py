"""Pins of the CPU oracle (CPU only): each check ties it to SDPA, a closed
form, brute force, an identity or a hand-worked fixture."""
import json
import os

import pytest

import oracle
import oracle_checks as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle)


def test_paging_fixture():
    with open(os.path.join(GOLDEN, "paging_fixture.json")) as f:
        fx = json.load(f)
    oc.check_paging_fixture(oracle, fx)
