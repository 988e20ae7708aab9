"""The seeded input generator: shapes, determinism, formats, distributions."""
import numpy as np

import synth


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0 ** -130, 3.0e38], dtype=np.float32)
    b = synth.bf16_bits(x)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 tie -> up to 1+2^-6... (mantissa 7 bits)
    assert b[0] == 0x3F80 and b[1] == 0x3F80 and b[2] == 0x3F82
    assert np.array_equal(synth.bf16_from_bits(b)[:3], np.array([1.0, 1.0, 1.0 + 2 ** -6], np.float32))


def test_dictionary_unit_norm_and_deterministic():
    D1 = synth.make_dictionary(np.random.default_rng(5), 256, 128, "bf16")
    D2 = synth.make_dictionary(np.random.default_rng(5), 256, 128, "bf16")
    assert np.array_equal(D1, D2)
    n = np.linalg.norm(D1.astype(np.float64), axis=1)
    assert np.all(np.abs(n - 1) < 2 ** -7)
    assert np.array_equal(synth.bf16_round(D1), D1)  # values are bf16-exact


def test_codes_format():
    w = synth.make_codes(np.random.default_rng(6), 5000, 16, 32768)
    idx = (w & 0xFFFF).astype(np.int64)
    coef = (w >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    assert idx.max() < 32768
    s = np.sort(idx, axis=1)
    assert not (s[:, 1:] == s[:, :-1]).any()           # distinct atoms per vector
    assert (coef >= 0).all() and (np.diff(coef, axis=1) <= 0).all()  # |N(0,1)| descending


def test_decode_case_shapes():
    c = synth.decode_case(B=2, Hq=4, Hkv=2, T=100, seed=9, n_atoms=512, d=64)
    assert c.q.shape == (2, 4, 64) and c.key_codes.shape == (2, 2, 100, 16)
    assert np.array_equal(c.key_low, c.key_codes[..., :3])
    assert c.m == 10
    assert np.array_equal(synth.bf16_round(c.q), c.q)


def test_tiny_case_recipe():
    t = synth.tiny_case(0)
    assert t["dk"].shape == (512, 64) and t["dk"].dtype == np.float32
    assert t["xk"].shape == (256, 64) and t["q"].shape == (1, 1, 64)
    # each key vector is 4 atoms + small noise: residual after removing them is small
    r = t["xk"] - np.einsum("nk,nkd->nd", t["coefs_k"], t["dk"][t["atoms_k"]])
    assert np.abs(r).std() < 0.02


def test_encode_case_recipe():
    e = synth.encode_case(seed=2, stream=0, n_vectors=64, n_atoms=1024)
    assert e.x.shape == (64, 128) and np.array_equal(synth.bf16_round(e.x), e.x)
    assert (np.diff(e.coefs, axis=1) <= 0).all()
