"""Pins of the oracle's integer-only softmax (oracle/integer_softmax.py) against
what mathematics and the published polynomial fix: the fixed-point constants
from exact integer arithmetic and a convergent series, the polynomial's
accuracy on its interval, a derived error bound of the integer exponential
over every INT16 input, a hand-worked two-token example, exact invariances,
and agreement with the float softmax."""
import math

import numpy as np
import pytest

import oracle
from oracle import integer_softmax as isx

P1 = 2.0 ** oracle.INT_SOFTMAX_P_BITS


def test_fixed_point_constants():
    # ln 2 = sum_{n>=1} 1 / (n 2^n); the tail after N terms is < 1 / 2^N
    from fractions import Fraction
    s = sum(Fraction(1, n * 2 ** n) for n in range(1, 80))
    assert math.floor(s * 2 ** 30) == isx.LN2_Q30 == math.floor((s + Fraction(1, 2 ** 79)) * 2 ** 30)
    assert isx.B_Q30 == (1353 << 30) // 1000
    assert isx.CA_Q30 == (344 * 10000 << 30) // (1000 * 3585)


def test_polynomial_fit_on_its_interval():
    # the published second-order fit a (p + b)^2 + c of exp on (-ln2, 0]
    p = np.linspace(-math.log(2), 0, 200001)
    a, b, c = 0.3585, 1.353, 0.344
    rel = np.abs(a * (p + b) ** 2 + c - np.exp(p)) / np.exp(p)
    assert 2.5e-3 < rel.max() < 3.2e-3  # the fit's known worst case, near p = -0.55


@pytest.mark.parametrize("k", [4, 8, 11, 14, 20, 30])
def test_int_exp_error_bound_all_inputs(k):
    """Every INT16-difference input qd in [-65534, 0] at shift k: the integer
    exponential times a 2^-2(k-g) equals exp(qd 2^-k) within the sum of the
    fit error (3.2e-3), the truncation of p to k bits (2^-k), the b and guard
    truncations (7 2^-kk) and the final floor (2^z / (0.5 2^2kk / a))."""
    c = isx.int_exp_consts(k)
    kk = k - c["g"]
    qd = np.arange(-65534, 1, dtype=np.int64)
    e = isx.int_exp(qd, c).astype(np.float64)
    approx = e * 0.3585 / 2.0 ** (2 * kk)
    x = qd / 2.0 ** k
    exact = np.exp(x)
    z = np.floor(-x / math.log(2) + 1e-12)
    keep = z <= 20
    bound = 1.1 * (3.2e-3 + 1.1 * 2.0 ** -k + 7 * 2.0 ** -kk + 0.72 * 2.0 ** (z - 2 * kk))
    rel = np.abs(approx - exact) / exact
    assert np.all(rel[keep] <= bound[keep]), (k, float((rel - bound)[keep].max()))
    assert np.all(e[z >= 32] == 0)


def test_two_token_worked_example():
    """s = (1, 0): k = 14, q = (16384, 0), q_b = 22167, q_c = 257578233.
    Second token: X = 16384 2^16 = 1073741824, z = 1, remainder 329480707,
    qp = -5027, t = 17140, L = 551357833, e = L >> 1 = 275678916. First:
    e = 22167^2 + q_c = 748954122. h = 2 -> (187238531, 68919729), sum
    256158260, r = floor(2^62 / sum) = 18003268832, p = (e r) >> 32 =
    (784850122, 288891701)."""
    p, info = oracle.int_softmax(np.array([1.0, 0.0], np.float32), return_info=True)
    assert info["k"] == 14 and info["q_b"] == 22167
    assert info["q_c"] == 257578233 and info["h"] == 2 and info["sum"] == 256158260
    assert info["r"] == 18003268832
    assert p.tolist() == [784850122, 288891701]
    assert abs(p[0] / p[1] - math.e) < 2e-3


def test_invariances_and_special_cases():
    rng = np.random.default_rng(5)
    # scores on a 2^-10 grid, so adding 0.25 below is exact in fp32
    s = (np.rint(rng.standard_normal(3000) * 2 * 1024) / 1024).astype(np.float32)
    s[0] = 7.5  # the largest |s| sets k = 12 (7.5 = 0.9375 2^3)
    p, info = oracle.int_softmax(s, return_info=True)
    assert info["k"] == 12
    # shifting every score by a multiple of 2^-k that keeps max|s| in its binade
    t = (s + np.float32(0.25)).astype(np.float32)
    assert np.array_equal(np.float64(t) - np.float64(s), np.full(s.size, 0.25))
    assert np.array_equal(oracle.int_softmax(t), p)
    # equal scores: equal probabilities summing to 1 within m units
    for m in (1, 2, 7, 13108):
        pe = oracle.int_softmax(np.full(m, -3.25, np.float32))
        assert np.all(pe == pe[0]) and abs(int(pe.sum()) - P1) <= m
    # a single token takes all of the mass
    assert oracle.int_softmax(np.array([0.1], np.float32))[0] in (P1 - 1, P1)
    # all-zero scores (k clamps to 30)
    pz = oracle.int_softmax(np.zeros(10, np.float32))
    assert np.all(pz == pz[0])


@pytest.mark.parametrize("scale", [0.0, 0.01, 1.0, 3.0, 30.0])
@pytest.mark.parametrize("m", [1, 5, 410, 13108])
def test_agrees_with_float_softmax(scale, m):
    rng = np.random.default_rng(int(scale * 100) + m)
    s = (rng.standard_normal(m) * scale).astype(np.float32)
    p = oracle.int_softmax(s)
    assert np.all(p >= 0)
    e = np.exp(s.astype(np.float64) - s.max())
    pf = e / e.sum()
    assert abs(p.sum() / P1 - 1.0) <= 2e-5
    d = np.abs(p / P1 - pf)
    assert np.all(d <= 0.02 * pf + 2.0 ** -16)
    assert d.sum() <= 2e-2


def test_decode_oracle_int_mode_close_to_float():
    import synth
    c = synth.decode_case(B=1, Hq=4, Hkv=2, T=300, seed=9, n_atoms=256)
    rf = oracle.decode_attn(c.q, c.dk, c.dv, c.key_codes, c.val_codes, c.klow, c.khigh,
                            c.top_num, c.top_den, c.scale)
    ri = oracle.decode_attn(c.q, c.dk, c.dv, c.key_codes, c.val_codes, c.klow, c.khigh,
                            c.top_num, c.top_den, c.scale, softmax="int")
    assert np.array_equal(rf["sel"], ri["sel"])
    assert np.allclose(ri["p"], ri["p_int"] / P1, rtol=0, atol=0)
    rel = np.linalg.norm(ri["out"] - rf["out"]) / np.linalg.norm(rf["out"])
    assert rel < 2e-2
    # with the float scores handed in explicitly the result is the same
    r2 = oracle.decode_attn(c.q, c.dk, c.dv, c.key_codes, c.val_codes, c.klow, c.khigh,
                            c.top_num, c.top_den, c.scale, sel=ri["sel"], softmax="int",
                            s_high_in=ri["s_high"].astype(np.float32))
    assert np.array_equal(r2["p_int"], ri["p_int"])
