"""The CPU oracle against its pins (hand-worked cases, the OCP FP8 spec,
torch's fp8/bf16 casts, closed forms, independent gather formulations)."""
import pytest

import oracle
import oracle_pins  # noqa: E402


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(orc, check):
    check(orc)
