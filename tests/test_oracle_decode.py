"""Pins of the oracle's hierarchical coded decode attention and top-k select
against closed forms, identities, brute force and a hand-worked fixture."""
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.DECODE_CHECKS, ids=lambda c: c.__name__)
def test_decode_pin(check):
    check(oracle.decode_attn)


def test_select_topk_bruteforce():
    pins.check_select_topk(oracle.select_topk)


def test_selected_count():
    assert oracle.selected_count(256, 1, 10) == 26      # ceil, not floor (25)
    assert oracle.selected_count(4096, 1, 10) == 410
    assert oracle.selected_count(131072, 1, 10) == 13108
    assert oracle.selected_count(32768, 1, 10) == 3277
    assert oracle.selected_count(262144, 1, 10) == 26215
    assert oracle.selected_count(1, 1, 10) == 1
    assert oracle.selected_count(7, 1, 1) == 7
