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


def test_prefill_encode_full_size_sampled():
    """The prefill encode workload at full size for the key stream (262,144
    bf16 vectors, 32,768 atoms, K=16) as the benchmark runs it; the oracle
    checks a seeded sample of 2,048 vectors."""
    H.log("encode prefill key stream (262144 vectors), oracle on 2048 sampled")
    e = synth.encode_case(stream=0)
    g = run(e.x, e.dictionary, 16)
    rng = np.random.default_rng(99)
    pick = np.sort(rng.choice(e.x.shape[0], 2048, replace=False))
    sub = {k: v[pick] for k, v in g.items()}
    compare(e.x[pick], e.dictionary, 16, sub, "prefill sample")
