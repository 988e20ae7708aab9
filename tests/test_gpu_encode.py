"""GPU parity of sdkv_encode (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as H
from tests import oracle_pins as pins

pytestmark = pytest.mark.gpu


def run(x, D, K, x_dtype="bf16", dict_dtype="bf16", klow=0):
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    xt = H.to_bf16(x) if x_dtype == "bf16" else H.to_f32(x)
    Dt = H.to_bf16(D) if dict_dtype == "bf16" else H.to_f32(D)
    r = sd.sdkv_encode(xt, Dt, K, coef_f32=True, resid_norm=True,
                       low_plane=bool(klow), klow=klow)
    torch.cuda.synchronize()
    return {k: H.host(v) for k, v in r.items()}


def compare(x, D, K, g, label):
    ri, rg, rn = oracle.mp_encode(x, D, K)
    gi, gc = H.unpack_words(g["codes"])
    agree = H.code_agreement(gi, ri)
    assert agree >= H.IDX_AGREE, f"{label}: index agreement {agree}"
    mask = H.matched_prefix_mask(gi, ri)
    cerr = np.abs(g["coef_f32"].astype(np.float64) - rg)[mask]
    assert cerr.size == 0 or cerr.max() <= H.COEF_TOL, f"{label}: coef err {cerr.max()}"
    perr = (np.abs(gc - rg) - H.f16_half_ulp(rg))[mask]
    assert perr.size == 0 or perr.max() <= H.COEF_TOL
    full = mask.all(axis=1)
    nerr = np.abs(g["resid_norm"].astype(np.float64) - rn)[full]
    assert nerr.size == 0 or nerr.max() <= 1e-4 * max(1.0, np.abs(rn).max())
    H.log(f"  {label}: n={x.shape[0]} idx agree {agree:.6f} coef err "
          f"{(cerr.max() if cerr.size else 0):.2e} vectors fully matched {full.mean():.4f}")
    return ri, rg, rn


def test_tiny_fp32_dictionary():
    H.log("encode tiny (fp32 dictionaries, d=64, K=4)")
    t = synth.tiny_case(0)
    for key, D in (("xk", t["dk"]), ("xv", t["dv"])):
        g = run(t[key], D, 4, x_dtype="f32", dict_dtype="f32")
        compare(t[key], D, 4, g, f"tiny {key}")


def test_exact_recovery_signed_permutation_bf16():
    """Exact recovery: signed permutation dictionary, exactly representable
    coefficients -> exact indices, coefficients and zero residual."""
    rng = np.random.default_rng(3)
    d, K, n = 128, 6, 700
    perm = rng.permutation(d)
    D = np.zeros((d, d), np.float32)
    D[np.arange(d), perm] = rng.choice([-1.0, 1.0], d)
    S = np.stack([rng.choice(d, K, replace=False) for _ in range(n)])
    c = np.array([8.0, -6.5, 4.25, -3.0, 1.5, -0.75], np.float32)
    x = np.einsum("k,nkd->nd", c, D[S])
    g = run(x, D, K)
    gi, _ = H.unpack_words(g["codes"])
    assert np.array_equal(gi, S)
    assert np.array_equal(g["coef_f32"], np.broadcast_to(c, (n, K)))
    assert np.all(g["resid_norm"] == 0)


def test_exact_recovery_erc_overcomplete():
    """Tropp's exact-recovery condition on a 512-atom fp32 dictionary."""
    rng = np.random.default_rng(4)
    D, S = pins.erc_dictionary(rng, 512, 64, 3)
    D = D.astype(np.float32)
    c = rng.standard_normal((200, 3)).astype(np.float32) * 2
    x = c @ D[S]
    g = run(x, D, 3, x_dtype="f32", dict_dtype="f32")
    gi, _ = H.unpack_words(g["codes"])
    order = np.argsort(-np.abs(c), axis=1)
    assert np.array_equal(gi, S[order])
    np.testing.assert_allclose(g["coef_f32"], np.take_along_axis(c, order, 1), atol=2e-5)


@pytest.mark.parametrize("n,N,K", [(1, 4096, 16), (100, 1000, 1), (513, 2048, 32),
                                   (1030, 32768, 16)])
def test_ragged_sizes(n, N, K):
    H.log(f"encode ragged n={n} N={N} K={K}")
    rng = np.random.default_rng(n + N + K)
    D = synth.make_dictionary(rng, N, 128, "bf16")
    x, _, _ = synth.make_sparse_vectors(rng, D, n, 16, 0.05, "absdesc")
    x = synth.bf16_round(x)
    g = run(x, D, K, klow=min(3, K))
    compare(x, D, K, g, f"n={n} N={N} K={K}")
    assert np.array_equal(g["low_plane"], g["codes"][:, :min(3, K)])


@pytest.mark.parametrize("n", [40, 200])
def test_max_atoms(n):
    """65,536 atoms, the largest dictionary the boundary takes (uint16
    indices; 4,096 16-atom tiles fill the batch screen's 12-bit tile field),
    on the small path (n <= 64) and the batch path."""
    H.log(f"encode n={n} N=65536")
    rng = np.random.default_rng(65536 + n)
    D = synth.make_dictionary(rng, 65536, 128, "bf16")
    x, _, _ = synth.make_sparse_vectors(rng, D, n, 16, 0.05, "absdesc")
    x = synth.bf16_round(x)
    g = run(x, D, 16)
    ri, _, _ = compare(x, D, 16, g, f"n={n} N=65536")
    assert ri.max() >= 32768   # atoms in the upper half are picked


def test_head_dim_64_bf16():
    rng = np.random.default_rng(21)
    D = synth.make_dictionary(rng, 3000, 64, "bf16")
    x, _, _ = synth.make_sparse_vectors(rng, D, 900, 8, 0.02, "normal")
    x = synth.bf16_round(x)
    compare(x, D, 8, run(x, D, 8), "d=64")


def test_deterministic():
    rng = np.random.default_rng(22)
    D = synth.make_dictionary(rng, 4096, 128, "bf16")
    x = synth.bf16_round(rng.standard_normal((600, 128), dtype=np.float32))
    a, b = run(x, D, 16), run(x, D, 16)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def near_tie_case(rng, n, N=4096, d=128, winner_high=True):
    """Vectors whose two largest correlations belong to atoms a < b of the
    same 16-atom column (a = b mod 16, b in a higher tile), apart by a
    relative 2^-12 .. 2^-15: below what an fp16 screen resolves. x = d_a +
    d_b + e (d_w - d_l) in fp32, w the intended winner (b when
    winner_high). Returns (x, D, a, b) after checking in fp64 that the two
    lead and how far apart they are."""
    D = synth.make_dictionary(rng, N, d, "bf16")
    ntile = N // 16
    c = rng.integers(0, 16, n)
    t1 = rng.integers(0, ntile - 1, n)
    t2 = t1 + 1 + (rng.integers(0, ntile, n) % (ntile - 1 - t1))
    a, b = 16 * t1 + c, 16 * t2 + c
    eps = 2.0 ** -rng.uniform(12, 15, n)
    w, lo = (b, a) if winner_high else (a, b)
    # x = alpha d_lo + beta d_w with <x, d_lo> = 1 and <x, d_w> = 1 + eps
    # (fp64 solve of the 2x2 Gram system), stored in fp32
    Dl, Dw = D[lo].astype(np.float64), D[w].astype(np.float64)
    gll, gww, glw = (Dl * Dl).sum(1), (Dw * Dw).sum(1), (Dl * Dw).sum(1)
    det = gll * gww - glw * glw
    tl, tw = np.ones(n), 1.0 + eps
    alpha = (gww * tl - glw * tw) / det
    beta = (gll * tw - glw * tl) / det
    x = (alpha[:, None] * Dl + beta[:, None] * Dw).astype(np.float32)
    C = x.astype(np.float64) @ D.T.astype(np.float64)
    top2 = np.argsort(-np.abs(C), axis=1)[:, :2]
    assert np.array_equal(top2[:, 0], w), "construction: intended winner is not first"
    assert np.array_equal(top2[:, 1], lo), "construction: partner is not second"
    gap = (np.abs(C[np.arange(n), w]) - np.abs(C[np.arange(n), lo])) / np.abs(C[np.arange(n), w])
    assert np.all(gap > 2.0 ** -17) and np.all(gap < 2.0 ** -11), gap
    return x, D, a, b


@pytest.mark.parametrize("n", [1030, 48])
@pytest.mark.parametrize("winner_high", [True, False])
def test_near_ties_within_one_screen_column(n, winner_high):
    """The two best atoms share a screen column and differ by less than the
    fp16 screen resolves: the exact pick must still find the larger one
    (batch path n > 64 and the small path), at every step."""
    H.log(f"encode near ties in one column n={n} winner_high={winner_high}")
    rng = np.random.default_rng(500 + n + winner_high)
    x, D, a, b = near_tie_case(rng, n, winner_high=winner_high)
    g = run(x, D, 2, x_dtype="f32")
    gi, _ = H.unpack_words(g["codes"])
    ri, rg, _ = oracle.mp_encode(x, D, 2)
    assert np.array_equal(ri[:, 0], b if winner_high else a)
    bad = np.nonzero((gi != ri).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} vectors differ, first {bad[:5]}: gpu {gi[bad[:3]]} oracle {ri[bad[:3]]}"
    np.testing.assert_allclose(g["coef_f32"], rg, atol=H.COEF_TOL, rtol=0)


def exact_tie_dictionary(rng, N=8192, d=128):
    """A bf16 dictionary with exact ties: rows copied or negated onto other
    rows of the same screen column and of other columns, and three equal
    rows in one column (which the exact pick must rescan). Returns
    (D, groups): each group lists rows whose |<x, d>| are all equal."""
    D = synth.make_dictionary(rng, N, d, "bf16")
    groups = []
    for j in range(40):
        base = 16 * (2 * j + 1) + (j % 16)
        if j % 4 == 0:      # copy in the same column, higher tile
            others = [base + 16 * (50 + j)]
        elif j % 4 == 1:    # negated copy in the same column
            others = [base + 16 * (60 + j)]
        elif j % 4 == 2:    # copy in another column
            others = [base + 16 * (70 + j) + 3]
        else:               # three equal rows in one column
            others = [base + 16 * (80 + j), base + 16 * (150 + j)]
        sign = -1.0 if j % 4 == 1 else 1.0
        assert all(o < N for o in others)
        for o in others:
            D[o] = sign * D[base]
        groups.append([base] + others)
    rows = [r for gr in groups for r in gr]
    assert len(set(rows)) == len(rows)
    return D, groups


@pytest.mark.parametrize("n", [1000, 40])
def test_exact_ties_take_the_lowest_atom(n):
    """Vectors aligned with rows that have exact duplicates (copied or
    negated, in the same screen column or not, up to three in a column):
    equal |correlations|, and the lowest atom index must win, as in the
    oracle (numpy's argmax takes the first maximum)."""
    H.log(f"encode exact ties n={n}")
    rng = np.random.default_rng(600 + n)
    D, groups = exact_tie_dictionary(rng)
    gsel = rng.integers(0, len(groups), n)
    heads = np.array([groups[k][0] for k in gsel])
    x = (2.0 * D[heads] + 0.01 * rng.standard_normal((n, 128))).astype(np.float32)
    g = run(x, D, 3, x_dtype="f32")
    gi, _ = H.unpack_words(g["codes"])
    ri, rg, _ = oracle.mp_encode(x, D, 3)
    assert np.array_equal(ri[:, 0], heads)
    bad = np.nonzero((gi != ri).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} vectors differ, first {bad[:5]}: gpu {gi[bad[:3]]} oracle {ri[bad[:3]]}"
    np.testing.assert_allclose(g["coef_f32"], rg, atol=H.COEF_TOL, rtol=0)


@pytest.mark.slow
@pytest.mark.parametrize("stream", [0, 1])
def test_prefill_encode_full_size_sampled(stream):
    """The prefill encode workload at full size for the key (0) and value (1)
    stream (262,144 bf16 vectors each, 32,768 atoms, K=16) as the benchmark
    runs it; the oracle checks a seeded sample of 16,384 vectors of each."""
    H.log(f"encode prefill stream {stream} (262144 vectors), oracle on 16384 sampled")
    e = synth.encode_case(stream=stream)
    g = run(e.x, e.dictionary, 16)
    rng = np.random.default_rng(99 + stream)
    pick = np.sort(rng.choice(e.x.shape[0], 16384, replace=False))
    sub = {k: v[pick] for k, v in g.items()}
    compare(e.x[pick], e.dictionary, 16, sub, f"prefill stream {stream} sample")


def random_encode_shape(seed):
    """A seeded random encode problem: vector counts on the small path
    (n <= 64) and the batch path, dictionaries from 17 to 12,000 atoms,
    head dims 64/128, code lengths 1 to 32, bf16 or fp32 inputs and
    dictionaries, with and without the low plane."""
    rng = np.random.default_rng(9400 + seed)
    return dict(n=int(rng.choice([33, 64, 65, 300, 1500])),
                N=int(rng.choice([17, 1000, 4096, 12000])),
                d=int(rng.choice([64, 128])), K=int(rng.integers(1, 33)),
                x_dtype=str(rng.choice(["bf16", "f32"])),
                dict_dtype=str(rng.choice(["bf16", "f32"])),
                klow=int(rng.integers(0, 5)), seed=1100 + seed)


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(seed):
    s = random_encode_shape(seed)
    H.log(f"encode random shape {seed}: {s}")
    rng = np.random.default_rng(s["seed"])
    D = synth.make_dictionary(rng, s["N"], s["d"], s["dict_dtype"])
    # at most a quarter of the atoms in each vector (the distinct-index draw
    # rejects duplicates, which a near-full draw would take forever to avoid)
    x, _, _ = synth.make_sparse_vectors(rng, D, s["n"], min(16, s["N"] // 4), 0.05, "absdesc")
    if s["x_dtype"] == "bf16":
        x = synth.bf16_round(x)
    klow = min(s["klow"], s["K"])
    g = run(x, D, s["K"], x_dtype=s["x_dtype"], dict_dtype=s["dict_dtype"], klow=klow)
    compare(x, D, s["K"], g, f"random {seed}")
    if klow:
        assert np.array_equal(g["low_plane"], g["codes"][:, :klow])
