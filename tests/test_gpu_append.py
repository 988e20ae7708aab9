"""GPU parity of the decode-step append: the small-batch encode path
(n <= 64 vectors, fp32-accurate correlations spread over the device) against
the fp64 oracle, against the batch path, and written into a cache slot."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as H
from tests.test_gpu_encode import compare, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,N,K,d,dt", [(1, 32768, 16, 128, "bf16"), (16, 32768, 16, 128, "bf16"),
                                        (64, 1000, 8, 128, "bf16"), (5, 3000, 12, 64, "f32"),
                                        (33, 129, 32, 128, "bf16")])
def test_small_path_vs_oracle(n, N, K, d, dt):
    H.log(f"small-batch encode n={n} N={N} K={K} d={d} {dt}")
    rng = np.random.default_rng(1000 + n + N)
    D = synth.make_dictionary(rng, N, d, dt)
    x, _, _ = synth.make_sparse_vectors(rng, D, n, 16, 0.05, "absdesc")
    x = synth.bf16_round(x) if dt == "bf16" else x.astype(np.float32)
    g = run(x, D, K, x_dtype=dt, dict_dtype=dt, klow=min(3, K))
    compare(x, D, K, g, f"small n={n}")
    assert np.array_equal(g["low_plane"], g["codes"][:, :min(3, K)])


def test_small_path_exact_recovery():
    """Signed permutation dictionary: exact indices, coefficients, zero residual."""
    rng = np.random.default_rng(31)
    d, K, n = 128, 6, 40
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


def test_small_path_agrees_with_batch_path():
    """The same 64 vectors through the small path (n = 64) and inside a
    65-vector batch call (screen + exact recheck)."""
    rng = np.random.default_rng(32)
    D = synth.make_dictionary(rng, 32768, 128, "bf16")
    x, _, _ = synth.make_sparse_vectors(rng, D, 65, 16, 0.05, "absdesc")
    x = synth.bf16_round(x)
    small = run(x[:64], D, 16)
    batch = run(x, D, 16)
    si, _ = H.unpack_words(small["codes"])
    bi, _ = H.unpack_words(batch["codes"][:64])
    agree = H.code_agreement(si, bi)
    H.log(f"  small vs batch index agreement {agree:.6f}")
    assert agree >= H.IDX_AGREE


@pytest.mark.parametrize("n,N,K,d,dt", [(8, 32768, 16, 128, "bf16"), (64, 1000, 32, 128, "bf16"),
                                        (3, 777, 5, 64, "f32")])
def test_encode_pair_matches_two_single_encodes(n, N, K, d, dt):
    """sdkv_encode_pair (key and value problems in one launch sequence) gives
    each side exactly what sdkv_encode gives it alone: codes, fp32
    coefficients, residual norms and low plane, bit for bit; the key input is
    bf16 and the value input fp32."""
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    H.log(f"encode pair n={n} N={N} K={K} d={d} {dt}")
    rng = np.random.default_rng(500 + n)
    Dk = synth.make_dictionary(rng, N, d, dt)
    Dv = synth.make_dictionary(rng, N, d, dt)
    xk, _, _ = synth.make_sparse_vectors(rng, Dk, n, 16, 0.05, "absdesc")
    xv, _, _ = synth.make_sparse_vectors(rng, Dv, n, 16, 0.05, "absdesc")
    xk = synth.bf16_round(xk)
    xv = xv.astype(np.float32)
    conv = H.to_bf16 if dt == "bf16" else H.to_f32
    Dkt, Dvt, xkt, xvt = conv(Dk), conv(Dv), H.to_bf16(xk), H.to_f32(xv)
    klow = min(3, K)
    out = {}
    for side in ("k", "v"):
        out[side] = dict(codes=torch.full((n, K), -1, dtype=torch.int32, device="cuda"),
                         coef=torch.full((n, K), float("nan"), dtype=torch.float32, device="cuda"),
                         rn=torch.full((n,), float("nan"), dtype=torch.float32, device="cuda"),
                         low=torch.full((n, klow), -1, dtype=torch.int32, device="cuda"))

    def args(side, x, D):
        o = out[side]
        return sd.EncodeArgs(x=x.data_ptr(), x_dtype=sd.SDKV_BF16 if x.dtype == torch.bfloat16 else sd.SDKV_F32,
                             dict=D.data_ptr(), dict_dtype=sd.SDKV_BF16 if D.dtype == torch.bfloat16 else sd.SDKV_F32,
                             n=n, d=d, n_atoms=N, K=K, codes=o["codes"].data_ptr(),
                             coef_f32=o["coef"].data_ptr(), resid_norm=o["rn"].data_ptr(),
                             low_plane=o["low"].data_ptr(), klow=klow)
    ws = sd.Workspace()
    sd.sdkv_encode_pair(args("k", xkt, Dkt), args("v", xvt, Dvt), ws)
    torch.cuda.synchronize()
    for side, x, D, xt in (("k", xk, Dk, xkt), ("v", xv, Dv, xvt)):
        ref = sd.sdkv_encode(xt, Dkt if side == "k" else Dvt, K, coef_f32=True, resid_norm=True,
                             low_plane=True, klow=klow)
        torch.cuda.synchronize()
        o = out[side]
        assert np.array_equal(H.host(o["codes"]), H.host(ref["codes"])), side
        assert np.array_equal(H.host(o["coef"]), H.host(ref["coef_f32"])), side
        assert np.array_equal(H.host(o["rn"]), H.host(ref["resid_norm"])), side
        assert np.array_equal(H.host(o["low"]), H.host(ref["low_plane"])), side
        compare(x, D, K, {"codes": H.host(o["codes"]), "coef_f32": H.host(o["coef"]),
                          "resid_norm": H.host(o["rn"])}, f"pair {side}")


@pytest.mark.parametrize("interleaved", [True, False])
def test_append_into_cache_slot(interleaved):
    """One decode step's new keys and values (B=2, Hkv=4) encoded into slot
    t = 17 of a 50-token cache: the slot holds exactly the codes a plain
    encode gives, the key low plane its first words, and nothing else in the
    cache changes."""
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    rng = np.random.default_rng(33)
    B, Hkv, T, K, d, t, klow = 2, 4, 50, 16, 128, 17, 3
    dk = synth.make_dictionary(rng, 4096, d, "bf16")
    dv = synth.make_dictionary(rng, 4096, d, "bf16")
    xk, _, _ = synth.make_sparse_vectors(rng, dk, B * Hkv, 16, 0.05, "absdesc")
    xv, _, _ = synth.make_sparse_vectors(rng, dv, B * Hkv, 16, 0.05, "absdesc")
    xk, xv = synth.bf16_round(xk), synth.bf16_round(xv)
    fill = rng.integers(0, 2**31 - 1, size=(B, Hkv, T, 2, K), dtype=np.int64).astype(np.int32)
    low0 = rng.integers(0, 2**31 - 1, size=(B, Hkv, T, klow), dtype=np.int64).astype(np.int32)
    dkt, dvt = H.to_bf16(dk), H.to_bf16(dv)
    xkt, xvt = H.to_bf16(xk).reshape(B, Hkv, d), H.to_bf16(xv).reshape(B, Hkv, d)
    low = torch.from_numpy(low0.copy()).cuda()
    if interleaved:
        kv = torch.from_numpy(fill.copy()).cuda()
        sd.sdkv_append_tokens(xkt, xvt, dkt, dvt, kv, None, t, key_low=low)
        torch.cuda.synchronize()
        got = H.host(kv)
        gk, gv = got[:, :, :, 0, :], got[:, :, :, 1, :]
        fk, fv = fill[:, :, :, 0, :], fill[:, :, :, 1, :]
    else:
        kc = torch.from_numpy(np.ascontiguousarray(fill[:, :, :, 0, :])).cuda()
        vc = torch.from_numpy(np.ascontiguousarray(fill[:, :, :, 1, :])).cuda()
        sd.sdkv_append_tokens(xkt, xvt, dkt, dvt, kc, vc, t, key_low=low)
        torch.cuda.synchronize()
        gk, gv = H.host(kc), H.host(vc)
        fk, fv = fill[:, :, :, 0, :], fill[:, :, :, 1, :]
    gl = H.host(low)
    other = np.ones(T, bool)
    other[t] = False
    assert np.array_equal(gk[:, :, other], fk[:, :, other])
    assert np.array_equal(gv[:, :, other], fv[:, :, other])
    assert np.array_equal(gl[:, :, other], low0[:, :, other])
    ref_k = run(xk, dk, K)["codes"].reshape(B, Hkv, K)
    ref_v = run(xv, dv, K)["codes"].reshape(B, Hkv, K)
    assert np.array_equal(gk[:, :, t], ref_k)
    assert np.array_equal(gv[:, :, t], ref_v)
    assert np.array_equal(gl[:, :, t], ref_k[:, :, :klow])
    # and the codes match the oracle's pursuit
    ri, _, _ = oracle.mp_encode(xk, dk, K)
    gi, _ = H.unpack_words(ref_k.reshape(-1, K))
    assert H.code_agreement(gi, ri) >= H.IDX_AGREE
