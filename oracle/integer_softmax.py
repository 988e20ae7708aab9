"""Integer-only softmax over a row of attention scores (fp64 oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: review page, Summary (the integer-only contribution: integer
polynomial approximations for Softmax; Softmax inputs requantized to
token-wise INT16; bit-shift guards against INT32 overflow; fixed-point
reciprocals for the divisions) and Strengths (Table 1 and Section 3.1.3:
token-wise INT16 requantization is what keeps the integer nonlinearities from
diverging). The polynomial is the second-order fit of exp on (-ln2, 0] that
the integer-only BERT work (I-BERT) uses, exp(p) ~ a (p + b)^2 + c with
a = 0.3585, b = 1.353, c = 0.344, after writing x = -z ln2 + p so that
exp(x) = 2^-z exp(p).

Readings (the pages give no formulas; each choice is stated in the design doc):
  * "token-wise" = one scale per softmax row (one query token and head).
    The scale is a power of two, 2^-k with k = 15 - E where the row's
    largest |score| is f 2^E (f in [0.5, 1)), clamped to k in [1, 30]; so
    the requantization is a shift and every constant below is an exact
    function of k. q_t = clamp(rint(s_t 2^k), -32767, 32767).
  * q_t - max_t q_t enters the exponential (so every input is <= 0).
  * The constants ln2, b and c/a are fixed-point integers with 30
    fractional bits (floor). The range reduction x = -z ln2 + p runs at 30
    fractional bits (so z ln2 carries no truncation error that grows with
    z); b and c/a are shifted to the row's precision.
  * Bit-shift guards: the polynomial is evaluated at min(k, 14) fractional
    bits (the squared term then stays below 2^31), and the exponentials are
    shifted right, rounding half up, by h = max(0, bitlen(m) + bitlen(max e)
    - 30) before they are summed, so the INT32 sum stays below 2^30 + m <
    2^31. (Rounding rather than truncating keeps the m-term sum unbiased; a
    truncating shift loses up to m units, which at m ~ 10^4 tokens is a
    visible share of the mass.)
  * Fixed-point reciprocal: r = floor(2^62 / sum), at least 31 significant
    bits; p_t = (e_t r) >> 32 is the probability with 30 fractional bits
    (p in [0, 2^30]); e_t r <= 2^62 since e_t <= sum.

Everything after the fp32 scores is integer arithmetic (Python ints via
int64 NumPy arrays, all values < 2^62), so another implementation that is
handed the same fp32 scores must reproduce p bit for bit.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = ["int_softmax", "INT_SOFTMAX_P_BITS", "int_exp_consts"]

A_POLY = Fraction(3585, 10000)
B_POLY = Fraction(1353, 1000)
C_POLY = Fraction(344, 1000)
Q = 30                                       # fractional bits of the constants
LN2_Q30 = math.floor(math.log(2.0) * 2 ** Q)  # fractional part ~0.95: fp64 is exact enough
B_Q30 = math.floor(B_POLY * 2 ** Q)
CA_Q30 = math.floor(C_POLY / A_POLY * 2 ** Q)
IN_BITS = 15                                 # INT16 magnitude
K_MIN, K_MAX = 1, 30
POLY_BITS = 14                               # precision cap of the polynomial
INT_SOFTMAX_P_BITS = 30


def _bitlen(x: int) -> int:
    return int(x).bit_length()


def int_exp_consts(k: int) -> dict:
    """Row constants at input precision 2^-k: q_b = floor(b 2^k), the guard
    shift g of the polynomial, and q_c = floor((c/a) 2^(2(k-g))) (each from
    its 30-bit constant by a right shift)."""
    g = max(0, k - POLY_BITS)
    kk = k - g
    return {"k": k, "q_b": B_Q30 >> (Q - k), "g": g, "q_c": CA_Q30 >> (Q - 2 * kk)}


def row_shift(s: np.ndarray) -> int:
    """k: the power-of-two requantization shift of a row of fp32 scores."""
    amax = float(np.max(np.abs(s))) if s.size else 0.0
    if amax == 0.0:
        return K_MAX
    _, E = math.frexp(amax)                  # amax = f 2^E, f in [0.5, 1)
    return min(K_MAX, max(K_MIN, IN_BITS - E))


def int_exp(qd: np.ndarray, c: dict) -> np.ndarray:
    """Integer exponential of inputs qd <= 0 (scale 2^-k). The range
    reduction runs at 30 fractional bits: X = -qd 2^(30-k), z = floor(X /
    ln2_30), and p = -(X - z ln2_30) / 2^30 in (-ln2, 0] is truncated to k
    bits (qp); then 2^-z times the polynomial at qp; zero once z >= 31."""
    k = c["k"]
    X = (-np.asarray(qd, dtype=np.int64)) << (Q - k)
    z = X // LN2_Q30
    qp = -((X - z * LN2_Q30) >> (Q - k))
    t = (qp + c["q_b"]) >> c["g"]
    L = t * t + c["q_c"]
    return np.where(z >= 31, 0, L >> np.minimum(z, 62))


def int_softmax(scores, *, return_info: bool = False):
    """p_t (int64, 30 fractional bits) for one row of fp32 scores."""
    s = np.asarray(scores, dtype=np.float32).astype(np.float64)
    m = s.size
    k = row_shift(s)
    c = int_exp_consts(k)
    q = np.clip(np.rint(np.ldexp(s, k)), -32767, 32767).astype(np.int64)
    e = int_exp(q - q.max(), c)
    maxe = ((c["q_b"] >> c["g"]) ** 2) + c["q_c"]
    h = max(0, _bitlen(m) + _bitlen(maxe) - 30)
    e2 = (e + (1 << (h - 1))) >> h if h > 0 else e
    tot = int(e2.sum())
    assert 0 < tot < 2 ** 31
    r = (1 << 62) // tot
    p = (e2 * r) >> 32
    if return_info:
        return p, {"k": k, "h": h, "sum": tot, "r": r, "q": q, "e": e2, **c}
    return p
