"""Pin checks for the fp64 oracle, written as functions of the encode /
decode implementation under test so that the same checks can be run against
deliberately broken copies (tests/test_oracle_mutants.py).

Each check pins the oracle to something other than itself: a closed form,
an invariant of the mathematics, exact rational brute force on tiny inputs,
or a hand-worked fixture under tests/golden/.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f16_words(idx, coef):
    """Pack index/coefficient pairs (test-side, independent of the oracle)."""
    i = np.asarray(idx, dtype=np.uint32)
    c = np.asarray(coef, dtype=np.float16).view(np.uint16).astype(np.uint32)
    return (i | (c << 16)).astype(np.uint32)


# ---------------------------------------------------------------------------
# Encode pins
# ---------------------------------------------------------------------------
def check_golden_mp(encode):
    g = load_golden("mp_worked_example.json")
    D = np.array(g["dictionary"], dtype=np.float64)
    x = np.array([g["x"]], dtype=np.float64)
    idx, gam, rn = encode(x, D, g["K"])
    assert list(idx[0]) == g["idx"], (idx[0], g["idx"])
    assert np.array_equal(gam[0], np.array(g["gamma"])), (gam[0], g["gamma"])
    assert abs(rn[0] ** 2 - g["resid_norm_sq"]) < 1e-15, rn[0] ** 2


def orthonormal_dictionary(rng, d):
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return Q.T.copy()  # rows orthonormal


def check_exact_recovery_orthonormal(encode, seed=11):
    """Tropp's exact-recovery condition holds trivially for an orthonormal
    basis: the pursuit must pick the support in decreasing |c| order, return
    the true coefficients and leave a zero residual."""
    rng = np.random.default_rng(seed)
    d, K = 32, 6
    D = orthonormal_dictionary(rng, d)
    for _ in range(20):
        S = rng.choice(d, K, replace=False)
        mags = rng.uniform(0.5, 3.0, K) + 0.25 * rng.permutation(K)
        c = rng.choice([-1.0, 1.0], K) * mags
        x = c @ D[S]
        idx, gam, rn = encode(x[None], D, K)
        order = np.argsort(-np.abs(c))
        assert list(idx[0]) == list(S[order])
        np.testing.assert_allclose(gam[0], c[order], rtol=0, atol=1e-12)
        assert rn[0] < 1e-12


def check_exact_recovery_signed_permutation(encode, seed=12):
    """Signed permutation of the identity (exact in bf16): exact recovery
    with bit-exact coefficients."""
    rng = np.random.default_rng(seed)
    d, K = 16, 5
    perm = rng.permutation(d)
    signs = rng.choice([-1.0, 1.0], d)
    D = np.zeros((d, d))
    D[np.arange(d), perm] = signs
    S = rng.choice(d, K, replace=False)
    c = np.array([4.0, -3.5, 2.25, -1.5, 0.75])
    x = c @ D[S]
    idx, gam, rn = encode(x[None], D, K)
    assert list(idx[0]) == list(S)
    assert np.array_equal(gam[0], c)
    assert rn[0] == 0.0


def erc_dictionary(rng, n_atoms, d, K):
    """Overcomplete dictionary whose first K atoms are orthonormal and whose
    other atoms are unit Gaussian, redrawn until Tropp's exact-recovery
    condition max_{a not in S} sum_{i in S} |<d_i, d_a>| < 1 holds."""
    Q, _ = np.linalg.qr(rng.standard_normal((d, K)))
    supp = Q.T
    rest = rng.standard_normal((n_atoms - K, d))
    rest /= np.linalg.norm(rest, axis=1, keepdims=True)
    while True:
        erc = np.abs(rest @ supp.T).sum(axis=1)
        bad = erc >= 0.9
        if not bad.any():
            break
        r = rng.standard_normal((int(bad.sum()), d))
        rest[bad] = r / np.linalg.norm(r, axis=1, keepdims=True)
    D = np.concatenate([supp, rest])
    perm = rng.permutation(n_atoms)
    Dp = D[perm]
    S = np.argsort(perm)[:K]  # where the support atoms landed
    return Dp, S


def check_exact_recovery_erc(encode, seed=13):
    rng = np.random.default_rng(seed)
    d, K, N = 64, 3, 512
    D, S = erc_dictionary(rng, N, d, K)
    others = np.setdiff1d(np.arange(N), S)
    assert (np.abs(D[others] @ D[S].T).sum(axis=1) < 1).all()
    for _ in range(10):
        c = rng.standard_normal(K) * 2
        x = c @ D[S]
        idx, gam, rn = encode(x[None], D, K)
        order = np.argsort(-np.abs(c))
        assert list(idx[0]) == list(S[order])
        np.testing.assert_allclose(gam[0], c[order], atol=1e-12)
        assert rn[0] < 1e-12


def check_energy_identity(encode_trace, seed=14):
    """|r_{k+1}|^2 = |r_k|^2 - g_k^2 (2 - |d_{a_k}|^2) at every step, for
    atoms of any norm; for unit atoms the energy falls by g_k^2."""
    rng = np.random.default_rng(seed)
    d, N, K = 24, 80, 7
    D = rng.standard_normal((N, d))
    D *= rng.uniform(0.5, 1.3, (N, 1)) / np.linalg.norm(D, axis=1, keepdims=True)
    X = rng.standard_normal((40, d))
    idx, gam, rn, tr = encode_trace(X, D, K)
    dn2 = (D ** 2).sum(axis=1)
    lhs = tr[:, 1:] ** 2
    rhs = tr[:, :-1] ** 2 - gam ** 2 * (2 - dn2[idx])
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-10)


def check_telescoping_and_orthogonality(encode, seed=15):
    """Unit atoms: |x|^2 = sum_k g_k^2 + |r_K|^2, the final residual equals
    x - sum_k g_k d_{a_k}, and it is orthogonal to the last atom picked."""
    rng = np.random.default_rng(seed)
    d, N, K = 32, 200, 9
    D = rng.standard_normal((N, d))
    D /= np.linalg.norm(D, axis=1, keepdims=True)
    X = rng.standard_normal((30, d))
    idx, gam, rn = encode(X, D, K)
    np.testing.assert_allclose((X ** 2).sum(1), (gam ** 2).sum(1) + rn ** 2, rtol=1e-12)
    R = X - np.einsum("nk,nkd->nd", gam, D[idx])
    np.testing.assert_allclose(np.linalg.norm(R, axis=1), rn, rtol=1e-9, atol=1e-12)
    last = D[idx[:, -1]]
    assert np.abs((R * last).sum(1)).max() < 1e-12


def check_bruteforce_exact(encode, seed=16):
    """Exact rational brute force on tiny integer inputs (ties included):
    every step's atom is the first one maximising |<r, d_a>|, found by
    exhaustive search in Fraction arithmetic."""
    rng = np.random.default_rng(seed)
    for trial in range(30):
        d, N, K = 4, 9, 4
        D = rng.integers(-2, 3, (N, d)).astype(np.float64)
        D[rng.integers(0, N)] = 0.0
        D[1] = D[0] * -1  # a guaranteed |c| tie between atoms 0 and 1
        D[4] = 1.0 if trial % 2 else D[4]
        x = rng.integers(-4, 5, d).astype(np.float64)
        r = [Fraction(int(v)) for v in x]
        Dq = [[Fraction(int(v)) for v in row] for row in D]
        exp_idx, exp_g = [], []
        for _ in range(K):
            best, ba = Fraction(-1), -1
            cs = []
            for a in range(N):
                c = sum(ri * di for ri, di in zip(r, Dq[a]))
                cs.append(c)
                if abs(c) > best:
                    best, ba = abs(c), a
            g = cs[ba]
            r = [ri - g * di for ri, di in zip(r, Dq[ba])]
            exp_idx.append(ba)
            exp_g.append(g)
        idx, gam, rn = encode(x[None], D, K)
        assert list(idx[0]) == exp_idx, (trial, list(idx[0]), exp_idx)
        for k in range(K):
            if exp_g[k].denominator < 2 ** 20:
                assert abs(gam[0, k] - float(exp_g[k])) <= 1e-9 * max(1, abs(float(exp_g[k])))


def check_k1_is_argmax(encode, seed=17):
    """K = 1 reduces to: the first atom of largest |<x, d_a>|, coefficient
    <x, d_a>; compared against an exhaustive loop with math.fsum."""
    rng = np.random.default_rng(seed)
    D = rng.standard_normal((300, 16))
    D /= np.linalg.norm(D, axis=1, keepdims=True)
    X = rng.standard_normal((25, 16))
    idx, gam, _ = encode(X, D, 1)
    for n in range(X.shape[0]):
        cs = [math.fsum(X[n] * D[a]) for a in range(D.shape[0])]
        best = max(range(len(cs)), key=lambda a: (abs(cs[a]), -a))
        assert idx[n, 0] == best
        assert abs(gam[n, 0] - cs[best]) < 1e-12


ENCODE_CHECKS = [check_golden_mp, check_exact_recovery_orthonormal,
                 check_exact_recovery_signed_permutation,
                 check_exact_recovery_erc, check_telescoping_and_orthogonality,
                 check_bruteforce_exact, check_k1_is_argmax]


# ---------------------------------------------------------------------------
# Decode pins
# ---------------------------------------------------------------------------
# --- OMP (the comparison encoder) ---------------------------------------------
def check_omp_equals_mp_on_orthonormal(omp, mp, seed=40):
    """On an orthonormal dictionary the least-squares refit returns the
    projection coefficients, so OMP and the pursuit agree: same atoms,
    coefficients within 1e-12. K = 1 agrees on any dictionary."""
    rng = np.random.default_rng(seed)
    D = orthonormal_dictionary(rng, 24)
    X = rng.standard_normal((6, 24))
    i1, g1, r1 = omp(X, D, 7)
    i2, g2, r2 = mp(X, D, 7)
    assert np.array_equal(i1, i2)
    np.testing.assert_allclose(g1, g2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r1, r2, rtol=0, atol=1e-12)
    D2 = rng.standard_normal((40, 12))
    D2 /= np.linalg.norm(D2, axis=1, keepdims=True)
    i1, g1, _ = omp(X[:, :12], D2, 1)
    i2, g2, _ = mp(X[:, :12], D2, 1)
    assert np.array_equal(i1, i2)
    np.testing.assert_allclose(g1, g2, rtol=0, atol=1e-12)


def check_omp_refit_properties(omp, seed=41):
    """The final residual is orthogonal to every selected atom, equals x
    minus the coded reconstruction, and the residual norm never grows from
    one step to the next (least squares over a larger support)."""
    rng = np.random.default_rng(seed)
    D = rng.standard_normal((300, 32))
    D /= np.linalg.norm(D, axis=1, keepdims=True)
    X = rng.standard_normal((5, 32))
    idx, gam, rn, tr = omp(X, D, 10, trace=True)
    for v in range(5):
        r = X[v] - gam[v] @ D[idx[v]]
        assert abs(np.linalg.norm(r) - rn[v]) < 1e-12
        assert np.abs(D[idx[v]] @ r).max() < 1e-12
        assert np.all(np.diff(tr[v]) <= 1e-12)
        assert len(set(idx[v].tolist())) == 10


def check_omp_exact_recovery_coherent_support(omp, mp, seed=42):
    """A 3-atom support with pairwise inner products of 0.3 and every other
    atom satisfying Tropp's exact-recovery condition for OMP,
    |pinv(D_S) d_a|_1 < 1: OMP picks exactly the support, returns the true
    coefficients and a zero residual in 3 steps. The pursuit, without the
    refit, leaves a nonzero residual on the same input."""
    rng = np.random.default_rng(seed)
    d, K, N = 48, 3, 200
    G = np.full((K, K), 0.3) + 0.7 * np.eye(K)
    L = np.linalg.cholesky(G)
    Q, _ = np.linalg.qr(rng.standard_normal((d, K)))
    supp = (Q @ L.T).T  # rows with Gram matrix G
    rest = rng.standard_normal((N - K, d))
    rest /= np.linalg.norm(rest, axis=1, keepdims=True)
    pinv = np.linalg.pinv(supp.T)
    while True:
        bad = np.abs(rest @ pinv.T).sum(axis=1) >= 0.9
        if not bad.any():
            break
        r = rng.standard_normal((int(bad.sum()), d))
        rest[bad] = r / np.linalg.norm(r, axis=1, keepdims=True)
    D = np.concatenate([supp, rest])
    for _ in range(8):
        c = rng.uniform(0.5, 2.0, K) * rng.choice([-1.0, 1.0], K)
        x = c @ supp
        idx, gam, rn = omp(x[None], D, K)
        assert sorted(idx[0].tolist()) == [0, 1, 2]
        np.testing.assert_allclose(gam[0], c[idx[0]], rtol=0, atol=1e-12)
        assert rn[0] < 1e-12
        assert mp(x[None], D, K)[2][0] > 1e-3


def check_omp_bruteforce_rational(omp, seed=43):
    """Tiny integer inputs in exact rational arithmetic: first atom of
    largest |<r, d_a>| (ties to the lower index), then the exact
    least-squares coefficients from the normal equations by Gaussian
    elimination over the rationals."""
    from fractions import Fraction as F
    rng = np.random.default_rng(seed)
    for _ in range(6):
        d, N, K = 4, 7, 3
        Dn = rng.integers(-3, 4, (N, d)).astype(np.float64)
        Dn[np.all(Dn == 0, axis=1)] = 1.0
        x = rng.integers(-5, 6, d).astype(np.float64)
        Dq = [[F(int(v)) for v in row] for row in Dn]
        xq = [F(int(v)) for v in x]
        r = list(xq)
        S, g = [], []
        for _k in range(K):
            c = [sum(a * b for a, b in zip(Dq[i], r)) for i in range(N)]
            best = max(abs(ci) for ci in c)
            S.append(next(i for i in range(N) if abs(c[i]) == best))
            M = [[sum(a * b for a, b in zip(Dq[i], Dq[j])) for j in S] + [sum(a * b for a, b in zip(Dq[i], xq))]
                 for i in S]
            k = len(S)
            for col in range(k):  # Gauss-Jordan over the rationals
                piv = next(rw for rw in range(col, k) if M[rw][col] != 0)
                M[col], M[piv] = M[piv], M[col]
                M[col] = [v / M[col][col] for v in M[col]]
                for rw in range(k):
                    if rw != col and M[rw][col] != 0:
                        f = M[rw][col]
                        M[rw] = [a - f * b for a, b in zip(M[rw], M[col])]
            g = [M[i][k] for i in range(k)]
            r = [xq[t] - sum(g[i] * Dq[S[i]][t] for i in range(k)) for t in range(d)]
        idx, gam, _ = omp(x[None], Dn, K)
        assert list(idx[0]) == S, (list(idx[0]), S)
        np.testing.assert_allclose(gam[0], [float(v) for v in g], rtol=1e-12, atol=1e-12)


def check_omp_exact_fit(omp, seed=44):
    """Once the residual is exactly zero (the exact-fit reading): a zero
    vector gives atom 0 with coefficient 0 in every slot; x = 3 e_2 over the
    standard basis of R^8 is fitted by atom 2 with coefficient 3, after which
    atom 0 fills the remaining slots with coefficient 0 (worked by hand)."""
    rng = np.random.default_rng(seed)
    D = rng.standard_normal((40, 16))
    D /= np.linalg.norm(D, axis=1, keepdims=True)
    idx, gam, rn = omp(np.zeros((1, 16)), D, 4)
    assert idx.tolist() == [[0, 0, 0, 0]] and np.all(gam == 0) and rn[0] == 0
    x = np.zeros((1, 8))
    x[0, 2] = 3.0
    idx, gam, rn = omp(x, np.eye(8), 4)
    assert idx.tolist() == [[2, 0, 0, 0]], idx
    assert gam.tolist() == [[3.0, 0.0, 0.0, 0.0]], gam
    assert rn[0] == 0


OMP_CHECKS = [check_omp_refit_properties, check_omp_bruteforce_rational, check_omp_exact_fit]


def reconstruct(words, D, n_slots):
    """Explicit vectors sum_{j<n_slots} coef_j * D[idx_j] built with plain
    loops (independent of the oracle's table lookups)."""
    T = words.shape[0]
    out = np.zeros((T, D.shape[1]))
    for t in range(T):
        for j in range(n_slots):
            w = int(words[t, j])
            i = w & 0xFFFF
            c = float(np.array([w >> 16], dtype=np.uint16).view(np.float16)[0])
            out[t] += c * D[i]
    return out


def small_decode_inputs(seed, B=1, Hq=2, Hkv=1, T=40, N=24, d=8, K=4):
    rng = np.random.default_rng(seed)
    dk = rng.standard_normal((N, d)); dk /= np.linalg.norm(dk, axis=1, keepdims=True)
    dv = rng.standard_normal((N, d)); dv /= np.linalg.norm(dv, axis=1, keepdims=True)
    idx = rng.integers(0, N, (B, Hkv, T, K))
    kc = f16_words(idx, rng.standard_normal((B, Hkv, T, K)))
    vc = f16_words(rng.integers(0, N, (B, Hkv, T, K)), rng.standard_normal((B, Hkv, T, K)))
    q = rng.standard_normal((B, Hq, d))
    return q, dk, dv, kc, vc


def check_golden_decode(decode):
    g = load_golden("decode_worked_example.json")
    D = np.array(g["dictionary"], dtype=np.float64)
    kc = f16_words(np.array([[p[0] for p in t] for t in g["key_codes"]]),
                   np.array([[p[1] for p in t] for t in g["key_codes"]]))
    vc = f16_words(np.array([[p[0] for p in t] for t in g["val_codes"]]),
                   np.array([[p[1] for p in t] for t in g["val_codes"]]))
    q = np.array(g["q"], dtype=np.float64)[None, None]
    r = decode(q, D, D, kc[None, None], vc[None, None], g["klow"], g["khigh"],
               g["top_num"], g["top_den"], g["scale"])
    for key in ("u", "s_low", "s_high", "p", "w", "out"):
        assert np.array_equal(r[key][0, 0], np.array(g[key])), (key, r[key][0, 0], g[key])
    assert list(r["sel"][0, 0]) == g["sel"]


def check_dense_reduction(decode, seed=21):
    """Top fraction 100% and Klow = Khigh = K: textbook softmax attention over
    the explicitly reconstructed keys and values."""
    q, dk, dv, kc, vc = small_decode_inputs(seed, Hq=3, Hkv=3)
    K = kc.shape[-1]
    scale = 0.37
    r = decode(q, dk, dv, kc, vc, K, K, 1, 1, scale)
    for h in range(3):
        Kh = reconstruct(kc[0, h], dk, K)
        Vh = reconstruct(vc[0, h], dv, K)
        logits = [scale * math.fsum(Kh[t] * q[0, h]) for t in range(Kh.shape[0])]
        mx = max(logits)
        e = [math.exp(l - mx) for l in logits]
        z = math.fsum(e)
        o = sum((e[t] / z) * Vh[t] for t in range(len(e)))
        np.testing.assert_allclose(r["out"][0, h], o, rtol=1e-10, atol=1e-12)


def check_score_identities(decode, seed=22):
    """s_low[t] = scale <q, first-klow reconstruction of k_t>; s_high the same
    with khigh, on the selected tokens; out = sum_t p_t v_t and
    w-contraction agree; p is a softmax of s_high."""
    q, dk, dv, kc, vc = small_decode_inputs(seed, Hq=2, Hkv=1, T=50, K=5)
    klow, khigh, scale = 2, 4, 0.8
    r = decode(q, dk, dv, kc, vc, klow, khigh, 3, 10, scale)
    Klo = reconstruct(kc[0, 0], dk, klow)
    Khi = reconstruct(kc[0, 0], dk, khigh)
    V = reconstruct(vc[0, 0], dv, kc.shape[-1])
    for h in range(2):
        np.testing.assert_allclose(r["s_low"][0, h], scale * (Klo @ q[0, h]), atol=1e-12)
        S = r["sel"][0, h]
        np.testing.assert_allclose(r["s_high"][0, h], scale * (Khi[S] @ q[0, h]), atol=1e-12)
        sh = r["s_high"][0, h]
        p = np.exp(sh - sh.max()); p /= p.sum()
        np.testing.assert_allclose(r["p"][0, h], p, atol=1e-14)
        assert abs(r["p"][0, h].sum() - 1) < 1e-14
        np.testing.assert_allclose(r["out"][0, h], (r["p"][0, h][:, None] * V[S]).sum(0), atol=1e-12)


def check_selection_rule(decode, seed=23):
    """The selected set: m = ceil(T*num/den) tokens, ascending, the largest
    s_low with ties to the lower index (checked by a Python sort on
    (-score, index) tuples), including constructed exact ties."""
    q, dk, dv, kc, vc = small_decode_inputs(seed, T=37, K=3)
    kc = kc.copy()
    kc[0, 0, 10:20] = kc[0, 0, 3]  # ten tokens with identical codes -> ties
    r = decode(q, dk, dv, kc, vc, 2, 3, 1, 4, 1.0)
    m = r["m"]
    assert m == -(-37 // 4) == 10
    for h in range(q.shape[1]):
        s = r["s_low"][0, h]
        want = sorted(sorted(range(37), key=lambda t: (-s[t], t))[:m])
        assert list(r["sel"][0, h]) == want


def check_closed_forms(decode, seed=24):
    """m = 1: output is the value of the single best token. Identical key
    codes everywhere: every score ties, the first m tokens are taken and the
    output is the mean of their values."""
    q, dk, dv, kc, vc = small_decode_inputs(seed, T=30, K=3)
    r = decode(q, dk, dv, kc, vc, 2, 3, 1, 1000, 1.0)
    assert r["m"] == 1
    V = reconstruct(vc[0, 0], dv, 3)
    for h in range(q.shape[1]):
        t = int(np.argmax(r["s_low"][0, h]))
        np.testing.assert_allclose(r["out"][0, h], V[t], atol=1e-12)
    kc2 = np.broadcast_to(kc[:, :, :1], kc.shape).copy()
    r2 = decode(q, dk, dv, kc2, vc, 2, 3, 1, 3, 1.0)
    m = r2["m"]
    assert m == 10
    for h in range(q.shape[1]):
        assert list(r2["sel"][0, h]) == list(range(m))
        np.testing.assert_allclose(r2["out"][0, h], V[:m].mean(0), atol=1e-12)


def check_gqa_mapping(decode, seed=25):
    """Query head h reads KV head h // G (contiguous groups): each query head's
    result equals a single-head call on its own KV head."""
    q, dk, dv, kc, vc = small_decode_inputs(seed, B=2, Hq=6, Hkv=2, T=20, K=3)
    r = decode(q, dk, dv, kc, vc, 1, 3, 1, 2, 0.5)
    for b in range(2):
        for h in range(6):
            g = h // 3
            r1 = decode(q[b:b + 1, h:h + 1], dk, dv, kc[b:b + 1, g:g + 1],
                        vc[b:b + 1, g:g + 1], 1, 3, 1, 2, 0.5)
            np.testing.assert_array_equal(r["out"][b, h], r1["out"][0, 0])
            np.testing.assert_array_equal(r["sel"][b, h], r1["sel"][0, 0])


def check_kv_shared_selection(decode, seed=27):
    """select="kv": (a) one query head per KV head reduces to per-head
    selection; (b) identical queries within a group give the per-head
    result; (c) queries q and -q in a group of two cancel exactly, every
    shared score is 0 and the first m tokens are taken; (d) the shared score
    is the sum of the group's per-head low scores, every head of a group
    takes the same set, and that set is the top m of the sum under the
    (-score, index) order."""
    q, dk, dv, kc, vc = small_decode_inputs(seed, B=2, Hq=3, Hkv=3, T=33, K=4)
    a = decode(q, dk, dv, kc, vc, 2, 4, 1, 4, 0.7)
    k = decode(q, dk, dv, kc, vc, 2, 4, 1, 4, 0.7, select="kv")
    for key in ("sel", "s_low", "out"):
        np.testing.assert_array_equal(a[key], k[key])
    q2, dk, dv, kc, vc = small_decode_inputs(seed + 1, B=1, Hq=4, Hkv=2, T=29, K=3)
    q2[:, 1], q2[:, 3] = q2[:, 0], q2[:, 2]
    a = decode(q2, dk, dv, kc, vc, 2, 3, 1, 3, 1.0)
    k = decode(q2, dk, dv, kc, vc, 2, 3, 1, 3, 1.0, select="kv")
    np.testing.assert_array_equal(a["sel"], k["sel"])
    np.testing.assert_allclose(k["out"], a["out"], rtol=0, atol=1e-14)
    q3 = q2.copy()
    q3[:, 1], q3[:, 3] = -q3[:, 0], -q3[:, 2]
    k = decode(q3, dk, dv, kc, vc, 2, 3, 1, 3, 1.0, select="kv")
    assert np.all(k["s_low"] == 0.0)
    for h in range(4):
        assert list(k["sel"][0, h]) == list(range(k["m"]))
    q4, dk, dv, kc, vc = small_decode_inputs(seed + 2, B=2, Hq=6, Hkv=2, T=41, K=4)
    a = decode(q4, dk, dv, kc, vc, 3, 4, 2, 7, 0.8)
    k = decode(q4, dk, dv, kc, vc, 3, 4, 2, 7, 0.8, select="kv")
    m = k["m"]
    for b in range(2):
        for g in range(2):
            hs = range(3 * g, 3 * g + 3)
            tot = sum(a["s_low"][b, h] for h in hs)
            want = sorted(sorted(range(41), key=lambda t: (-tot[t], t))[:m])
            for h in hs:
                np.testing.assert_allclose(k["s_low"][b, h], tot, rtol=0, atol=1e-12)
                assert list(k["sel"][b, h]) == want


def _textbook(q, Kt, Vt, scale):
    logits = [scale * math.fsum(Kt[t] * q) for t in range(Kt.shape[0])]
    mx = max(logits)
    e = [math.exp(l - mx) for l in logits]
    z = math.fsum(e)
    return sum((e[t] / z) * Vt[t] for t in range(len(e)))


def check_reading_b(decode, seed=28):
    """reading="B" (every token in the softmax): (a) with the top fraction at
    100% it equals reading A; (b) with Klow = Khigh = K it is textbook
    attention over all T tokens' explicit reconstructions, whatever m is;
    (c) in general it is textbook attention over per-token keys and values
    built from K pairs for the selected tokens and Klow pairs for the rest
    (reconstructed with plain loops)."""
    q, dk, dv, kc, vc = small_decode_inputs(seed, Hq=2, Hkv=1, T=23, K=4)
    a = decode(q, dk, dv, kc, vc, 2, 3, 1, 1, 0.6)
    r = decode(q, dk, dv, kc, vc, 2, 3, 1, 1, 0.6, reading="B")
    np.testing.assert_allclose(r["out"], a["out"], rtol=0, atol=1e-14)
    K = kc.shape[-1]
    r = decode(q, dk, dv, kc, vc, K, K, 1, 5, 0.6, reading="B")
    for h in range(2):
        o = _textbook(q[0, h], reconstruct(kc[0, 0], dk, K), reconstruct(vc[0, 0], dv, K), 0.6)
        np.testing.assert_allclose(r["out"][0, h], o, rtol=1e-10, atol=1e-12)
    klow, khigh = 2, 3
    r = decode(q, dk, dv, kc, vc, klow, khigh, 2, 7, 0.6, reading="B")
    for h in range(2):
        S = set(int(t) for t in r["sel"][0, h])
        Kl, Kh = reconstruct(kc[0, 0], dk, klow), reconstruct(kc[0, 0], dk, khigh)
        Vl, Vf = reconstruct(vc[0, 0], dv, klow), reconstruct(vc[0, 0], dv, K)
        Kt = np.array([Kh[t] if t in S else Kl[t] for t in range(23)])
        Vt = np.array([Vf[t] if t in S else Vl[t] for t in range(23)])
        np.testing.assert_allclose(r["out"][0, h], _textbook(q[0, h], Kt, Vt, 0.6),
                                   rtol=1e-10, atol=1e-12)


DECODE_CHECKS = [check_golden_decode, check_dense_reduction,
                 check_score_identities, check_selection_rule,
                 check_closed_forms, check_gqa_mapping, check_kv_shared_selection,
                 check_reading_b]


def check_select_topk(select, seed=26):
    rng = np.random.default_rng(seed)
    s = rng.integers(0, 6, (5, 40)).astype(np.float64)  # many exact ties
    for k in (1, 7, 40):
        got = select(s, k)
        for r in range(5):
            want = sorted(sorted(range(40), key=lambda t: (-s[r, t], t))[:k])
            assert list(got[r]) == want
