"""GPU parity of the OMP comparison encoder (SDKV_ENCODE_OMP, small path)
through the C ABI, against the fp64 oracle's omp_encode: indices, refit
coefficients and residual norms; exact recovery of a coherent support; the
key/value pair equal to two single encodes bit for bit; and the comparison
the encoder exists for (its residual against the pursuit's on the same
vectors)."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def run(x, D, K, algorithm="omp", klow=0):
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    r = sd.sdkv_encode(H.to_bf16(x), H.to_bf16(D), K, coef_f32=True, resid_norm=True,
                       low_plane=bool(klow), klow=klow, algorithm=algorithm)
    torch.cuda.synchronize()
    return {k: H.host(v) for k, v in r.items()}


def compare_omp(x, D, K, g, label):
    ri, rg, rn = oracle.omp_encode(x, D, K)
    gi, gc = H.unpack_words(g["codes"])
    agree = H.code_agreement(gi, ri)
    assert agree >= H.IDX_AGREE, f"{label}: index agreement {agree}"
    full = np.all(gi == ri, axis=1)
    cerr = np.abs(g["coef_f32"].astype(np.float64) - rg)[full]
    assert cerr.size == 0 or cerr.max() <= H.COEF_TOL, f"{label}: coef err {cerr.max()}"
    perr = (np.abs(gc - rg) - H.f16_half_ulp(rg))[full]
    assert perr.size == 0 or perr.max() <= H.COEF_TOL
    nerr = np.abs(g["resid_norm"].astype(np.float64) - rn)[full]
    assert nerr.size == 0 or nerr.max() <= 1e-4 * max(1.0, np.abs(rn).max())
    H.log(f"  {label}: n={x.shape[0]} idx agree {agree:.6f} coef err "
          f"{(cerr.max() if cerr.size else 0):.2e} vectors fully matched {full.mean():.4f}")
    return ri, rg, rn


@pytest.mark.parametrize("n,N,K,d", [(8, 32768, 16, 128), (64, 1000, 8, 128),
                                     (5, 3000, 12, 64), (33, 700, 32, 128)])
def test_omp_vs_oracle(n, N, K, d):
    H.log(f"OMP encode n={n} N={N} K={K} d={d}")
    rng = np.random.default_rng(2000 + n + N)
    D = synth.make_dictionary(rng, N, d, "bf16")
    x, _, _ = synth.make_sparse_vectors(rng, D, n, 16, 0.05, "absdesc")
    x = synth.bf16_round(x)
    g = run(x, D, K, klow=min(3, K))
    compare_omp(x, D, K, g, f"omp n={n}")
    assert np.array_equal(g["low_plane"], g["codes"][:, :min(3, K)])


def test_omp_exact_recovery_coherent_support():
    """Three bf16 atoms with pairwise inner products near 0.3, the rest of the
    dictionary under Tropp's condition for OMP: the support, its
    coefficients and a (numerically) zero residual in three steps."""
    rng = np.random.default_rng(44)
    d, K, N = 128, 3, 2048
    G = np.full((K, K), 0.3) + 0.7 * np.eye(K)
    Q, _ = np.linalg.qr(rng.standard_normal((d, K)))
    supp = synth.bf16_round((Q @ np.linalg.cholesky(G).T).T.astype(np.float32)).astype(np.float64)
    rest = rng.standard_normal((N - K, d))
    rest /= np.linalg.norm(rest, axis=1, keepdims=True)
    rest = synth.bf16_round(rest.astype(np.float32)).astype(np.float64)
    pinv = np.linalg.pinv(supp.T)
    assert (np.abs(rest @ pinv.T).sum(axis=1) < 0.9).all()
    D = np.concatenate([supp, rest])
    c = np.array([[1.5, -1.0, 0.75], [-0.5, 2.0, 1.25], [1.0, 1.0, -1.0]])
    x = (c @ supp).astype(np.float32)
    # x itself is not bf16-exact: feed the GPU fp32 inputs through the f32 path
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    r = sd.sdkv_encode(H.to_f32(x), H.to_bf16(D), K, coef_f32=True, resid_norm=True,
                       algorithm="omp")
    torch.cuda.synchronize()
    gi, _ = H.unpack_words(H.host(r["codes"]))
    gc = H.host(r["coef_f32"])
    for v in range(3):
        assert sorted(gi[v].tolist()) == [0, 1, 2]
        np.testing.assert_allclose(gc[v], c[v][gi[v]], atol=2e-5)
    assert H.host(r["resid_norm"]).max() < 1e-5


def test_omp_pair_equals_single_encodes():
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    rng = np.random.default_rng(45)
    n, N, K, d = 8, 4096, 16, 128
    Dk = synth.make_dictionary(rng, N, d, "bf16")
    Dv = synth.make_dictionary(rng, N, d, "bf16")
    xk = synth.bf16_round(synth.make_sparse_vectors(rng, Dk, n, 16, 0.05, "absdesc")[0])
    xv = synth.bf16_round(synth.make_sparse_vectors(rng, Dv, n, 16, 0.05, "absdesc")[0])
    outs = {}
    args = {}
    for side, x, D in (("k", xk, Dk), ("v", xv, Dv)):
        xt, Dt = H.to_bf16(x), H.to_bf16(D)
        o = dict(codes=torch.full((n, K), -1, dtype=torch.int32, device="cuda"),
                 coef=torch.full((n, K), float("nan"), dtype=torch.float32, device="cuda"),
                 rn=torch.full((n,), float("nan"), dtype=torch.float32, device="cuda"))
        outs[side] = (o, xt, Dt)
        args[side] = sd.EncodeArgs(x=xt.data_ptr(), x_dtype=sd.SDKV_BF16, dict=Dt.data_ptr(),
                                   dict_dtype=sd.SDKV_BF16, n=n, d=d, n_atoms=N, K=K,
                                   codes=o["codes"].data_ptr(), coef_f32=o["coef"].data_ptr(),
                                   resid_norm=o["rn"].data_ptr(), algorithm=sd.SDKV_ENCODE_OMP)
    sd.sdkv_encode_pair(args["k"], args["v"])
    torch.cuda.synchronize()
    for side in ("k", "v"):
        o, xt, Dt = outs[side]
        ref = sd.sdkv_encode(xt, Dt, K, coef_f32=True, resid_norm=True, algorithm="omp")
        torch.cuda.synchronize()
        assert np.array_equal(H.host(o["codes"]), H.host(ref["codes"])), side
        assert np.array_equal(H.host(o["coef"]), H.host(ref["coef_f32"])), side
        assert np.array_equal(H.host(o["rn"]), H.host(ref["resid_norm"])), side


def test_omp_residual_against_the_pursuit():
    """The comparison the encoder is kept for: on the same 64 vectors (16-atom
    combinations plus noise over a 32,768-atom dictionary), OMP's final
    residual is never above the pursuit's by more than rounding, and both
    match their oracles' mean residuals."""
    rng = np.random.default_rng(46)
    D = synth.make_dictionary(rng, 32768, 128, "bf16")
    x = synth.bf16_round(synth.make_sparse_vectors(rng, D, 64, 16, 0.05, "absdesc")[0])
    go = run(x, D, 16)
    gp = run(x, D, 16, algorithm="pursuit")
    _, _, rn_o = oracle.omp_encode(x, D, 16)
    _, _, rn_p = oracle.mp_encode(x, D, 16)
    assert abs(go["resid_norm"].mean() - rn_o.mean()) <= 1e-3 * rn_o.mean()
    assert abs(gp["resid_norm"].mean() - rn_p.mean()) <= 1e-3 * rn_p.mean()
    assert go["resid_norm"].mean() < gp["resid_norm"].mean()
    H.log(f"  mean |r_16|: OMP {go['resid_norm'].mean():.4f} (oracle {rn_o.mean():.4f}), "
          f"pursuit {gp['resid_norm'].mean():.4f} (oracle {rn_p.mean():.4f}), "
          f"|x| {np.linalg.norm(x, axis=1).mean():.4f}")


@pytest.mark.parametrize("n,algorithm", [(6, "omp"), (6, "pursuit"), (100, "pursuit")])
def test_zero_vectors(n, algorithm):
    """Zero vectors (every correlation zero): atom 0 with coefficient 0 in
    every slot and a zero residual norm, on the small path (n <= 64) for both
    encoders and on the batch path for the pursuit; the batch's other
    vectors as the oracle encodes them."""
    H.log(f"zero vectors: n={n} {algorithm}")
    rng = np.random.default_rng(47 + n)
    D = synth.make_dictionary(rng, 2048, 128, "bf16")
    x = synth.bf16_round(synth.make_sparse_vectors(rng, D, n, 16, 0.05, "absdesc")[0])
    z = [1, n - 2]
    x[z] = 0.0
    g = run(x, D, 8, algorithm=algorithm)
    gi, gc = H.unpack_words(g["codes"])
    assert np.all(gi[z] == 0) and np.all(gc[z] == 0)
    assert np.all(g["coef_f32"][z] == 0) and np.all(g["resid_norm"][z] == 0)
    if algorithm == "omp":
        compare_omp(x, D, 8, g, "omp with zero vectors")
    else:
        ri, _, rn = oracle.mp_encode(x, D, 8)
        assert H.code_agreement(gi, ri) >= H.IDX_AGREE
        assert np.abs(g["resid_norm"].astype(np.float64) - rn).max() <= 1e-4 * max(1.0, rn.max())
