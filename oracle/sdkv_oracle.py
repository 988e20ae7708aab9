"""fp64 oracle: matching-pursuit encode and hierarchical coded decode attention.

TEST INFRASTRUCTURE ONLY (see the package docstring). Everything is computed
in float64 from the exact values of the (bf16 / fp16 / fp32) inputs.
"""
from __future__ import annotations

import numpy as np

from oracle.integer_softmax import INT_SOFTMAX_P_BITS, int_softmax

__all__ = ["unpack_codes", "pack_codes", "mp_encode", "omp_encode", "decode_attn",
           "select_topk", "selected_count"]


# ---------------------------------------------------------------------------
# Code words
# ---------------------------------------------------------------------------
def unpack_codes(words: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Split packed 32-bit code words into (atom index int64, coefficient
    float64). Bits 0-15 hold the uint16 atom index, bits 16-31 the IEEE
    binary16 coefficient (review page, FAQ on the 15x figure: a vector is
    stored as the indices and coefficients of its atoms)."""
    w = np.asarray(words, dtype=np.uint32)
    idx = (w & np.uint32(0xFFFF)).astype(np.int64)
    coef = (w >> np.uint32(16)).astype(np.uint16).view(np.float16).astype(np.float64)
    return idx, coef


def pack_codes(idx: np.ndarray, coef: np.ndarray) -> np.ndarray:
    """Pack atom indices and coefficients into 32-bit words; the coefficient
    is rounded to binary16 with round-to-nearest-even (NumPy's float16 cast).
    Reading: the pursuit runs on unrounded coefficients and rounding happens
    only here, when the code is stored."""
    i = np.asarray(idx).astype(np.uint32)
    c = np.asarray(coef, dtype=np.float64).astype(np.float16)
    return (i | (c.view(np.uint16).astype(np.uint32) << np.uint32(16))).astype(np.uint32)


# ---------------------------------------------------------------------------
# Encode: projection-based greedy pursuit (matching pursuit, no refit)
# ---------------------------------------------------------------------------
def mp_encode(X: np.ndarray, D: np.ndarray, K: int, *, trace: bool = False,
              block: int = 512):
    """Greedy pursuit of each row of X over the atoms (rows) of D.

    Review page, Summary and Strengths: a greedy pursuit projects out one
    atom per step and, unlike OMP, never re-solves a least-squares problem.
    Per vector x:
        r_0 = x
        for k = 0 .. K-1:
            c_a   = <r_k, d_a>           for every atom a
            a_k   = smallest a with |c_a| maximal   (np.argmax takes the first)
            g_k   = c_{a_k}                          (projection coefficient)
            r_k+1 = r_k - g_k * d_{a_k}
    Readings (the pages are silent): the coefficient is <r, d> with no
    division by |d|^2 (atoms are unit-norm); an atom may be picked again;
    ties go to the lowest atom index; coefficients are kept unrounded during
    the pursuit.

    Vectors are independent, so rows are processed `block` at a time; each
    row goes through exactly the steps above.

    Returns (idx int64 [n,K], gamma float64 [n,K], resid_norm float64 [n]);
    with trace=True also the residual norms before each step [n, K+1].
    """
    X = np.asarray(X, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    n = X.shape[0]
    idx = np.zeros((n, K), dtype=np.int64)
    gam = np.zeros((n, K), dtype=np.float64)
    rn = np.zeros(n, dtype=np.float64)
    tr = np.zeros((n, K + 1), dtype=np.float64) if trace else None
    for s in range(0, n, block):
        e = min(n, s + block)
        R = X[s:e].copy()
        rows = np.arange(e - s)
        for k in range(K):
            if trace:
                tr[s:e, k] = np.linalg.norm(R, axis=1)
            C = R @ D.T
            a = np.argmax(np.abs(C), axis=1)
            g = C[rows, a]
            R = R - g[:, None] * D[a]
            idx[s:e, k] = a
            gam[s:e, k] = g
        rn[s:e] = np.linalg.norm(R, axis=1)
        if trace:
            tr[s:e, K] = rn[s:e]
    if trace:
        return idx, gam, rn, tr
    return idx, gam, rn


# ---------------------------------------------------------------------------
# Decode: two-level (Klow then Khigh) scoring over coded keys and values
def omp_encode(X: np.ndarray, D: np.ndarray, K: int, *, trace: bool = False):
    """Orthogonal matching pursuit: the comparison encoder that the pages'
    greedy pursuit replaces (review page, Summary and Strengths: the
    projection pursuit avoids OMP's least-squares refits). Per vector x:
        S = (), r_0 = x
        for k = 0 .. K-1:
            c_a  = <r_k, d_a>                 for every atom a
            a_k  = smallest a with |c_a| maximal
            S    = S + (a_k,)
            g    = argmin_g |x - sum_{j<=k} g_j d_{S_j}|^2   (least squares)
            r_k+1 = x - sum_{j<=k} g_j d_{S_j}
    The codes are the atoms in selection order with the final refit
    coefficients. Readings: the same tie rule as the pursuit; the least
    squares is solved from the normal equations with numpy.linalg.solve
    (the support's Gram matrix is nonsingular while its atoms are linearly
    independent, which the refit guarantees for k < d: a new atom with
    nonzero correlation to a residual orthogonal to the support lies outside
    its span). The pages leave the exact-fit case open; reading: once the
    residual is exactly zero every correlation is zero, the tie rule picks
    atom 0, and the fit is already exact, so that atom joins with
    coefficient 0 and no refit is made.

    Returns (idx int64 [n,K], gamma float64 [n,K] final coefficients,
    resid_norm float64 [n]); with trace=True also the residual norms before
    each step [n, K+1].
    """
    X = np.asarray(X, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    n = X.shape[0]
    idx = np.zeros((n, K), dtype=np.int64)
    gam = np.zeros((n, K), dtype=np.float64)
    rn = np.zeros(n, dtype=np.float64)
    tr = np.zeros((n, K + 1), dtype=np.float64) if trace else None
    for v in range(n):
        x = X[v]
        r = x.copy()
        S = []
        g = np.zeros(0)
        for k in range(K):
            if trace:
                tr[v, k] = np.linalg.norm(r)
            c = D @ r
            S.append(int(np.argmax(np.abs(c))))
            if not np.any(c):
                g = np.append(g, 0.0)
                continue
            DS = D[S]
            g = np.linalg.solve(DS @ DS.T, DS @ x)
            r = x - DS.T @ g
        idx[v] = S
        gam[v] = g
        rn[v] = np.linalg.norm(r)
        if trace:
            tr[v, K] = rn[v]
    if trace:
        return idx, gam, rn, tr
    return idx, gam, rn


# ---------------------------------------------------------------------------
def selected_count(T: int, top_num: int, top_den: int) -> int:
    """m = ceil(T * num / den) in integer arithmetic, clamped to [1, T].
    Reading of "the top 10%" (review page, Summary): a ceiling, never empty."""
    return max(1, min(T, -(-T * top_num // top_den)))


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of each row, ties to the lower index,
    returned in ascending index order. (The 'top 10%' step of the review
    page's Summary, as a stand-alone operation.)"""
    s = np.atleast_2d(np.asarray(scores, dtype=np.float64))
    out = np.zeros((s.shape[0], k), dtype=np.int64)
    for r in range(s.shape[0]):
        order = np.argsort(-s[r], kind="stable")
        out[r] = np.sort(order[:k])
    return out


def decode_attn(q, dk, dv, key_codes, val_codes, klow: int, khigh: int,
                top_num: int, top_den: int, scale: float, sel=None, softmax: str = "float",
                s_high_in=None, select: str = "head", reading: str = "A"):
    """Hierarchical coded decode attention for one layer.

    Review page, Summary: every token is scored from its first Klow atoms
    and the best tenth is rescored with Khigh atoms. FAQ: three atoms are
    enough to rank most tokens. Abstract page: keys and values are sums of
    fixed dictionary atoms, so <q, k_t> = sum_j kappa_tj <q, d_{i_tj}>.

    Inputs: q [B,Hq,d]; dk, dv [N,d]; key_codes, val_codes uint32
    [B,Hkv,T,K]. For each batch b and query head h (KV head g = h // G,
    G = Hq / Hkv):
        u      = scale * (Dk q_h)                         [N]
        s_low  = sum_{j<klow}  kappa_tj * u[i_tj]         every t < T
        S      = the m tokens with the largest s_low, ties to lower t,
                 m = ceil(T*num/den)
        s_high = sum_{j<khigh} kappa_tj * u[i_tj]         t in S
        p      = softmax over S of s_high
        w[a]   = sum_{t in S} p_t sum_{j<K} kappa^v_tj [i^v_tj == a]
        out_h  = Dv^T w
    Readings: the softmax runs over S only (unselected tokens are dropped);
    selection is per query head; the key code's first klow slots are the
    "low" atoms; values use all K slots; the scale multiplies the scores.

    `sel` (optional int [B,Hq,m]) replaces the selection step with a given
    selected set; everything after it is computed as above. The tests use it
    to re-evaluate the output on another implementation's selection when two
    selections differ only by tokens tied with the threshold.

    softmax="int" replaces p by the integer-only softmax of
    oracle.int_softmax (review page, Summary and Strengths: token-wise INT16
    requantization, integer polynomial exp, shift guards, fixed-point
    reciprocal) applied to s_high rounded to fp32, the precision in which
    the scores reach the requantization; p = p_int / 2^30 and w, out follow
    in fp64. `s_high_in` (optional [B,Hq,m], with `sel`) supplies those fp32
    scores instead, so the integer steps can be checked bit for bit on
    another implementation's scores. The result then also holds p_int.

    select="kv" shares one selection among the G query heads of a KV head
    (grouped-query attention): the tokens are ranked by the group's summed
    low score sum_{h in g} s_low_h = sum_{j<klow} kappa_tj U_g[i_tj] with
    U_g = sum_h u_h, and every head of the group takes the same S; s_high,
    p and w stay per head. Reading: the pages make the selection
    query-aware and say nothing of GQA (review page, Summary); summing the
    group's scores is the plainest shared ranking (the score of the
    group's summed query). In this mode res["s_low"] holds that shared
    ranking score for every head of the group.

    reading="B" lets every token into the softmax (the pages' other
    reading of "scores all tokens at Klow=3 and refines the top 10%":
    review page, Summary; FAQ): a selected token enters with s_high and all
    K value pairs, every other token with its own head's s_low and its first
    klow value pairs,
        p = softmax over all T of (s_high on S, s_low elsewhere)
        w[a] = sum_{t in S} p_t sum_{j<K} kappa^v_tj [i^v_tj == a]
             + sum_{t not in S} p_t sum_{j<klow} kappa^v_tj [i^v_tj == a].
    res["p"] keeps the selected tokens' probabilities. Reading B with the
    integer softmax is not defined here (nor in the library).

    Returns a dict of float64 arrays: u [B,Hq,N], s_low [B,Hq,T],
    sel int64 [B,Hq,m] ascending, s_high [B,Hq,m], p [B,Hq,m],
    w [B,Hq,N], out [B,Hq,d], and m.
    """
    q = np.asarray(q, dtype=np.float64)
    dk = np.asarray(dk, dtype=np.float64)
    dv = np.asarray(dv, dtype=np.float64)
    B, Hq, d = q.shape
    _, Hkv, T, K = key_codes.shape
    N = dk.shape[0]
    G = Hq // Hkv
    m = selected_count(T, top_num, top_den)
    res = {k: None for k in ("u", "s_low", "sel", "s_high", "p", "w", "out")}
    res["u"] = np.zeros((B, Hq, N))
    res["s_low"] = np.zeros((B, Hq, T))
    res["sel"] = np.zeros((B, Hq, m), dtype=np.int64)
    res["s_high"] = np.zeros((B, Hq, m))
    res["p"] = np.zeros((B, Hq, m))
    res["w"] = np.zeros((B, Hq, N))
    res["out"] = np.zeros((B, Hq, d))
    res["m"] = m
    if softmax == "int":
        res["p_int"] = np.zeros((B, Hq, m), dtype=np.int64)
    elif softmax != "float":
        raise ValueError(softmax)
    if select not in ("head", "kv"):
        raise ValueError(select)
    if reading not in ("A", "B") or (reading == "B" and softmax == "int"):
        raise ValueError((reading, softmax))
    for b in range(B):
        for g in range(Hkv):
            ki, kc = unpack_codes(key_codes[b, g])
            vi, vc = unpack_codes(val_codes[b, g])
            if select == "kv":
                u_g = sum(scale * (dk @ q[b, hh]) for hh in range(g * G, (g + 1) * G))
                s_shared = (kc[:, :klow] * u_g[ki[:, :klow]]).sum(axis=1)
            for h in range(g * G, (g + 1) * G):
                u = scale * (dk @ q[b, h])
                s_low = (kc[:, :klow] * u[ki[:, :klow]]).sum(axis=1)
                s_rank = s_shared if select == "kv" else s_low
                if sel is None:
                    order = np.argsort(-s_rank, kind="stable")
                    S = np.sort(order[:m])
                else:
                    S = np.sort(np.asarray(sel[b, h], dtype=np.int64))
                s_high = (kc[S, :khigh] * u[ki[S, :khigh]]).sum(axis=1)
                if softmax == "int":
                    s32 = (np.asarray(s_high_in[b, h], dtype=np.float32) if s_high_in is not None
                           else s_high.astype(np.float32))
                    pi = int_softmax(s32)
                    res["p_int"][b, h] = pi
                    p = pi.astype(np.float64) / 2.0 ** INT_SOFTMAX_P_BITS
                elif reading == "B":
                    rest = np.setdiff1d(np.arange(T), S)
                    s_all = np.concatenate([s_high, s_low[rest]])
                    e = np.exp(s_all - s_all.max())
                    p_all = e / e.sum()
                    p = p_all[:S.size]
                    p_rest = p_all[S.size:]
                else:
                    e = np.exp(s_high - s_high.max())
                    p = e / e.sum()
                w = np.bincount(vi[S].ravel(), weights=(p[:, None] * vc[S]).ravel(),
                                minlength=N)
                if reading == "B":
                    w = w + np.bincount(vi[rest, :klow].ravel(),
                                        weights=(p_rest[:, None] * vc[rest, :klow]).ravel(),
                                        minlength=N)
                res["u"][b, h] = u
                res["s_low"][b, h] = s_rank
                res["sel"][b, h] = S
                res["s_high"][b, h] = s_high
                res["p"][b, h] = p
                res["w"][b, h] = w
                res["out"][b, h] = dv.T @ w
    return res
