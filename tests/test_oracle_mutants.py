"""Planted mistakes: each mutant is the oracle's own source with one plausible
error written in (a flipped sign, a dropped term, a wrong index or count, a
different tie rule ...). Every mutant must fail at least one pin, which shows
the pins constrain the oracle rather than restate it. All of this runs on the
CPU and touches nothing outside a throw-away module namespace."""
import inspect
import types

import pytest

import oracle.sdkv_oracle as src_mod
from tests import oracle_pins as pins

SRC = inspect.getsource(src_mod)

ENCODE_MUTANTS = {
    "update_sign": ("R = R - g[:, None] * D[a]", "R = R + g[:, None] * D[a]"),
    "argmax_no_abs": ("a = np.argmax(np.abs(C), axis=1)", "a = np.argmax(C, axis=1)"),
    "ties_to_last": ("a = np.argmax(np.abs(C), axis=1)",
                     "a = C.shape[1] - 1 - np.argmax(np.abs(C)[:, ::-1], axis=1)"),
    "normalised_coef": ("g = C[rows, a]", "g = C[rows, a] / (D[a] ** 2).sum(axis=1)"),
    "stale_residual": ("C = R @ D.T", "C = X[s:e] @ D.T"),
    "one_step_short": ("for k in range(K):\n            if trace:",
                       "for k in range(K - 1):\n            if trace:"),
}

DECODE_MUTANTS = {
    "low_uses_khigh": ("s_low = (kc[:, :klow] * u[ki[:, :klow]])",
                       "s_low = (kc[:, :khigh] * u[ki[:, :khigh]])"),
    "high_uses_klow": ("s_high = (kc[S, :khigh] * u[ki[S, :khigh]])",
                       "s_high = (kc[S, :klow] * u[ki[S, :klow]])"),
    "floor_count": ("return max(1, min(T, -(-T * top_num // top_den)))",
                    "return max(1, min(T, T * top_num // top_den))"),
    "ties_to_higher": ('order = np.argsort(-s_rank, kind="stable")',
                       'order = (T - 1 - np.argsort(-s_rank[::-1], kind="stable"))'),
    "softmax_all_tokens": ("p = e / e.sum()",
                           "p = e / (e.sum() + np.exp(np.delete(s_low, S) - s_high.max()).sum())"),
    "no_scale": ("u = scale * (dk @ q[b, h])", "u = (dk @ q[b, h])"),
    "gqa_modulo": ("for h in range(g * G, (g + 1) * G):", "for h in range(g, Hq, Hkv):"),
    "values_khigh_only": ("w = np.bincount(vi[S].ravel(), weights=(p[:, None] * vc[S]).ravel(),",
                          "w = np.bincount(vi[S][:, :khigh].ravel(), weights=(p[:, None] * vc[S][:, :khigh]).ravel(),"),
    "unweighted_values": ("weights=(p[:, None] * vc[S]).ravel()", "weights=(vc[S] / len(S)).ravel()"),
    "value_dict_is_key_dict": ('res["out"][b, h] = dv.T @ w', 'res["out"][b, h] = dk.T @ w'),
    "kv_first_head_only": ("u_g = sum(scale * (dk @ q[b, hh]) for hh in range(g * G, (g + 1) * G))",
                           "u_g = scale * (dk @ q[b, g * G])"),
    "kv_strided_group": ("u_g = sum(scale * (dk @ q[b, hh]) for hh in range(g * G, (g + 1) * G))",
                         "u_g = sum(scale * (dk @ q[b, hh]) for hh in range(g, Hq, Hkv))"),
    "kv_own_score": ('s_rank = s_shared if select == "kv" else s_low', "s_rank = s_low"),
    "b_rest_scored_high": ("s_all = np.concatenate([s_high, s_low[rest]])",
                           "s_all = np.concatenate([s_high, (kc[rest, :khigh] * u[ki[rest, :khigh]]).sum(axis=1)])"),
    "b_rest_full_values": ("w = w + np.bincount(vi[rest, :klow].ravel(),\n                                        weights=(p_rest[:, None] * vc[rest, :klow]).ravel(),",
                           "w = w + np.bincount(vi[rest].ravel(),\n                                        weights=(p_rest[:, None] * vc[rest]).ravel(),"),
    "b_rest_outside_normaliser": ("p_all = e / e.sum()", "p_all = e / e[:S.size].sum()"),
}


def build(mutation):
    old, new = mutation
    assert old in SRC, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod


def _fails(checks, fn):
    for chk in checks:
        try:
            chk(fn)
        except Exception:
            return True
    return False


@pytest.mark.parametrize("name", sorted(ENCODE_MUTANTS))
def test_encode_mutant_is_caught(name):
    m = build(ENCODE_MUTANTS[name])
    caught = _fails(pins.ENCODE_CHECKS, lambda X, D, K: m.mp_encode(X, D, K))
    if not caught:
        try:
            pins.check_energy_identity(lambda X, D, K: m.mp_encode(X, D, K, trace=True))
        except Exception:
            caught = True
    assert caught, f"no pin catches encode mutant {name}"


@pytest.mark.parametrize("name", sorted(DECODE_MUTANTS))
def test_decode_mutant_is_caught(name):
    m = build(DECODE_MUTANTS[name])
    assert _fails(pins.DECODE_CHECKS, m.decode_attn), f"no pin catches decode mutant {name}"


def test_unmutated_source_passes():
    m = build(("import numpy as np", "import numpy as np"))
    assert not _fails(pins.DECODE_CHECKS, m.decode_attn)
    assert not _fails(pins.ENCODE_CHECKS, lambda X, D, K: m.mp_encode(X, D, K))


# --- the integer softmax -------------------------------------------------------
import math  # noqa: E402

import numpy as np  # noqa: E402

import oracle.integer_softmax as isx_mod  # noqa: E402

ISX_SRC = inspect.getsource(isx_mod)

INT_MUTANTS = {
    "guard_truncates": ("e2 = (e + (1 << (h - 1))) >> h if h > 0 else e", "e2 = e >> h"),
    "no_max_subtract": ("e = int_exp(q - q.max(), c)", "e = int_exp(np.minimum(q, 0), c)"),
    "short_reciprocal": ("r = (1 << 62) // tot\n    p = (e2 * r) >> 32",
                         "r = (1 << 31) // tot\n    p = (e2 * r) >> 1"),
    "b_shift_off_by_one": ('"q_b": B_Q30 >> (Q - k)', '"q_b": B_Q30 >> (Q - k - 1)'),
    "scale_off_by_one": ("return min(K_MAX, max(K_MIN, IN_BITS - E))",
                         "return min(K_MAX, max(K_MIN, IN_BITS - E + 1))"),
    "reduction_precision": ("qp = -((X - z * LN2_Q30) >> (Q - k))",
                            "qp = -((X - z * LN2_Q30) >> (Q - k + 1))"),
    "poly_sign": ('t = (qp + c["q_b"]) >> c["g"]', 't = (c["q_b"] - qp) >> c["g"]'),
}


def _int_checks(m):
    """The integer-softmax pins, run on module m."""
    def golden():
        assert m.int_softmax(np.array([1.0, 0.0], np.float32)).tolist() == [784850122, 288891701]

    def exp_bound():
        for k in (8, 14, 20):
            c = m.int_exp_consts(k)
            kk = k - c["g"]
            qd = np.arange(-40000, 1, dtype=np.int64)
            approx = m.int_exp(qd, c).astype(np.float64) * 0.3585 / 2.0 ** (2 * kk)
            x = qd / 2.0 ** k
            z = np.floor(-x / math.log(2) + 1e-12)
            keep = z <= 12
            bound = 1.1 * (3.2e-3 + 1.1 * 2.0 ** -k + 7 * 2.0 ** -kk + 0.72 * 2.0 ** (z - 2 * kk))
            assert np.all((np.abs(approx - np.exp(x)) / np.exp(x))[keep] <= bound[keep])

    def float_agreement():
        rng = np.random.default_rng(3)
        for scale, n in ((1.0, 410), (3.0, 2000), (0.01, 5000)):
            s = (rng.standard_normal(n) * scale).astype(np.float32)
            p = m.int_softmax(s) / 2.0 ** 30
            e = np.exp(s.astype(np.float64) - s.max())
            pf = e / e.sum()
            assert abs(p.sum() - 1) <= 2e-5 and np.abs(p - pf).sum() <= 2e-2

    return [golden, exp_bound, float_agreement]


def _int_fails(m):
    for chk in _int_checks(m):
        try:
            chk()
        except Exception:
            return True
    return False


def _build_isx(mutation):
    old, new = mutation
    assert old in ISX_SRC, old
    mod = types.ModuleType("isx_mutant")
    exec(compile(ISX_SRC.replace(old, new), "<isx-mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(INT_MUTANTS))
def test_int_softmax_mutant_is_caught(name):
    assert _int_fails(_build_isx(INT_MUTANTS[name])), f"no pin catches integer-softmax mutant {name}"


def test_unmutated_int_softmax_passes():
    assert not _int_fails(_build_isx(("import math", "import math")))


# --- the OMP comparison encoder -------------------------------------------------
OMP_MUTANTS = {
    "omp_no_refit": ("g = np.linalg.solve(DS @ DS.T, DS @ x)\n            r = x - DS.T @ g",
                     "g = np.append(g, c[S[-1]])\n            r = r - g[-1] * D[S[-1]]"),
    "omp_refit_on_residual": ("g = np.linalg.solve(DS @ DS.T, DS @ x)",
                              "g = np.linalg.solve(DS @ DS.T, DS @ r)"),
    "omp_ties_to_last": ("S.append(int(np.argmax(np.abs(c))))",
                         "S.append(int(len(c) - 1 - np.argmax(np.abs(c)[::-1])))"),
    "omp_drops_first_atom": ("DS = D[S]", "DS = D[S[1:] if len(S) > 1 else S]"),
}


@pytest.mark.parametrize("name", sorted(OMP_MUTANTS))
def test_omp_mutant_is_caught(name):
    m = build(OMP_MUTANTS[name])
    caught = False
    for chk in pins.OMP_CHECKS:
        try:
            chk(m.omp_encode)
        except Exception:
            caught = True
            break
    if not caught:
        try:
            pins.check_omp_exact_recovery_coherent_support(m.omp_encode, m.mp_encode)
        except Exception:
            caught = True
    assert caught, f"no pin catches OMP mutant {name}"
