"""Pins of the oracle's greedy pursuit (encode) against closed forms,
invariants, exact brute force and a hand-worked fixture."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def enc(X, D, K):
    return oracle.mp_encode(X, D, K)


def enc_trace(X, D, K):
    return oracle.mp_encode(X, D, K, trace=True)


@pytest.mark.parametrize("check", pins.ENCODE_CHECKS, ids=lambda c: c.__name__)
def test_encode_pin(check):
    check(enc)


def test_energy_identity():
    pins.check_energy_identity(enc_trace)


def test_block_independence():
    """Processing vectors in blocks does not change any vector's result."""
    rng = np.random.default_rng(3)
    D = rng.standard_normal((64, 8)); D /= np.linalg.norm(D, axis=1, keepdims=True)
    X = rng.standard_normal((37, 8))
    a = oracle.mp_encode(X, D, 5, block=512)
    b = oracle.mp_encode(X, D, 5, block=5)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_pack_roundtrip_and_rounding():
    """binary16 round-to-nearest-even at pack time; index in the low 16 bits."""
    idx = np.array([0, 1, 65535, 32767])
    coef = np.array([1.0 / 3.0, -2.5, 65504.0, 1.0 + 2.0 ** -11])
    w = oracle.pack_codes(idx, coef)
    assert list(w & 0xFFFF) == [0, 1, 65535, 32767]
    # 1/3 -> 0x3555 (RNE), -2.5 -> 0xC100, 65504 -> 0x7BFF, 1+2^-11 ties to even -> 0x3C00
    assert list(w >> 16) == [0x3555, 0xC100, 0x7BFF, 0x3C00]
    i2, c2 = oracle.unpack_codes(w)
    assert list(i2) == list(idx)
    assert c2[1] == -2.5 and c2[3] == 1.0
