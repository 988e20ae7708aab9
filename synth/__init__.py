"""Seeded synthetic inputs for the dictionary-coded KV cache.

This module only *draws* inputs: dictionaries, vectors to encode, queries and
pre-made codes in the packed 32-bit word format of the C library (low 16 bits:
atom index as uint16; high 16 bits: the coefficient's IEEE binary16 bits).
It contains none of the method's arithmetic (no pursuit, no scoring, no
selection, no softmax) and is shared by the tests, the benchmark and the
oracle's checks; neither the oracle nor the HIP library imports it.

Workload shapes follow the pages of "LLM Inference in a Flash!":
  * the review page (Summary; FAQ "What is the 15x KV cache compression")
    fixes K=16 atoms per vector, 32,768-atom per-layer, per-stream
    dictionaries, Klow=3, top 10% refined to Khigh=16;
  * the abstract names the Llama-3.1-8B and Qwen-2.5-7B models, whose
    attention shapes (32/8 and 28/4 query/KV heads, head_dim 128, 32 and 28
    layers) set the head counts used here.
The learned dictionaries, model weights and LongBench data are not available;
unit-normalised Gaussian atoms and random codes stand in for them.

Random draws use numpy's PCG64 (`numpy.random.default_rng`) in a fixed,
documented order so that every array is reproducible from its seed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "DecodeCase", "EncodeCase", "make_dictionary", "make_sparse_vectors",
    "make_codes", "make_query", "pack_words", "tiny_case", "decode_case",
    "encode_case", "DECODE_WORKLOADS", "bf16_round", "bf16_bits",
    "bf16_from_bits",
]


# --------------------------------------------------------------------------
# Plain number-format helpers (format conversion, not method arithmetic).
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the
    16-bit patterns as uint16."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    """Widen uint16 bfloat16 patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32 (exact value)."""
    return bf16_from_bits(bf16_bits(x))


def pack_words(idx: np.ndarray, coef_f16: np.ndarray) -> np.ndarray:
    """Pack (uint16 index, binary16 coefficient) pairs into uint32 words:
    index in bits 0-15, coefficient bits in 16-31."""
    i = np.asarray(idx).astype(np.uint32)
    c = np.asarray(coef_f16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    return (i | (c << 16)).astype(np.uint32)


# --------------------------------------------------------------------------
# Draws
# --------------------------------------------------------------------------
def make_dictionary(rng: np.random.Generator, n_atoms: int, d: int,
                    dtype: str = "bf16") -> np.ndarray:
    """Gaussian rows, normalised to unit length in float64, then cast.

    Returns float32 values (bf16-rounded when dtype == "bf16"); use
    `bf16_bits` to obtain the storage bits.
    """
    g = rng.standard_normal((n_atoms, d), dtype=np.float32).astype(np.float64)
    g /= np.linalg.norm(g, axis=1, keepdims=True)
    f = g.astype(np.float32)
    if dtype == "bf16":
        return bf16_round(f)
    if dtype == "f32":
        return f
    raise ValueError(dtype)


def _distinct_indices(rng: np.random.Generator, n: int, k: int,
                      n_atoms: int) -> np.ndarray:
    """n rows of k distinct uniform atom indices (rejection on duplicates)."""
    idx = rng.integers(0, n_atoms, size=(n, k), dtype=np.int64)
    if k == 1:
        return idx
    while True:
        s = np.sort(idx, axis=1)
        bad = np.nonzero((s[:, 1:] == s[:, :-1]).any(axis=1))[0]
        if bad.size == 0:
            return idx
        idx[bad] = rng.integers(0, n_atoms, size=(bad.size, k), dtype=np.int64)


def make_sparse_vectors(rng: np.random.Generator, D: np.ndarray, n: int,
                        k: int, noise_std: float, coef: str,
                        chunk: int = 65536) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """x = sum_j c_j * D[a_j] + N(0, noise_std^2) per row.

    coef == "normal":    c_j ~ N(0, 1)                      (tiny workload)
    coef == "absdesc":   c_j = |N(0,1)| sorted descending    (Llama-shaped)
    Returns (x float32 [n, d], atoms int64 [n, k], coefs float32 [n, k]).
    Draw order per call: atoms, coefficients, noise.
    """
    d = D.shape[1]
    atoms = _distinct_indices(rng, n, k, D.shape[0])
    c = rng.standard_normal((n, k), dtype=np.float32)
    if coef == "absdesc":
        c = -np.sort(-np.abs(c), axis=1)
    elif coef != "normal":
        raise ValueError(coef)
    noise = rng.standard_normal((n, d), dtype=np.float32) * np.float32(noise_std)
    x = np.empty((n, d), dtype=np.float32)
    D32 = D.astype(np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x[s:e] = np.einsum("nk,nkd->nd", c[s:e], D32[atoms[s:e]]) + noise[s:e]
    return x, atoms, c


def make_codes(rng: np.random.Generator, n: int, k: int,
               n_atoms: int) -> np.ndarray:
    """Pre-made codes: k distinct uniform indices and binary16 coefficients
    |N(0,1)| sorted in decreasing order (magnitude order, as a greedy pursuit
    emits them). Returns packed uint32 words [n, k]."""
    idx = _distinct_indices(rng, n, k, n_atoms)
    c = np.abs(rng.standard_normal((n, k), dtype=np.float32))
    c = -np.sort(-c, axis=1)
    return pack_words(idx, c.astype(np.float16))


def make_query(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16; returns float32 values."""
    return bf16_round(rng.standard_normal(shape, dtype=np.float32))


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------
@dataclass
class DecodeCase:
    """One decode-attention call's inputs (host arrays).

    q:        float32 [B, Hq, d]  (bf16-exact values)
    dk, dv:   float32 [N, d]      (bf16-exact values when dict_dtype == "bf16")
    key_codes, val_codes: uint32 [B, Hkv, T, K] packed words
    key_low:  uint32 [B, Hkv, T, klow] (first klow words of key_codes)
    """
    name: str
    q: np.ndarray
    dk: np.ndarray
    dv: np.ndarray
    key_codes: np.ndarray
    val_codes: np.ndarray
    key_low: np.ndarray
    K: int
    klow: int
    khigh: int
    top_num: int
    top_den: int
    scale: float
    dict_dtype: str = "bf16"
    extra: dict = field(default_factory=dict)

    @property
    def B(self): return self.q.shape[0]
    @property
    def Hq(self): return self.q.shape[1]
    @property
    def d(self): return self.q.shape[2]
    @property
    def Hkv(self): return self.key_codes.shape[1]
    @property
    def T(self): return self.key_codes.shape[2]
    @property
    def n_atoms(self): return self.dk.shape[0]

    @property
    def m(self) -> int:
        """Selected-token count: ceil(T * num / den), at least 1, at most T."""
        return max(1, min(self.T, -(-self.T * self.top_num // self.top_den)))


@dataclass
class EncodeCase:
    name: str
    x: np.ndarray          # float32 [n, d] (bf16-exact when x_dtype == "bf16")
    dictionary: np.ndarray # float32 [N, d]
    K: int
    x_dtype: str = "bf16"
    dict_dtype: str = "bf16"
    atoms: np.ndarray | None = None
    coefs: np.ndarray | None = None


def tiny_case(seed: int = 0) -> dict:
    """The tiny workload: one head, head_dim 64, 512-atom float32 key and
    value dictionaries, 256 tokens. Keys and values are 4-atom combinations
    with N(0,1) coefficients plus N(0, 0.01^2) noise; one bf16 query.

    Draw order: Dk, Dv, key vectors, value vectors, query.
    Returns a dict with the encode inputs; the decode codes are whatever an
    encoder makes of them (the caller encodes and packs).
    """
    rng = np.random.default_rng(seed)
    dk = make_dictionary(rng, 512, 64, "f32")
    dv = make_dictionary(rng, 512, 64, "f32")
    xk, ak, ck = make_sparse_vectors(rng, dk, 256, 4, 0.01, "normal")
    xv, av, cv = make_sparse_vectors(rng, dv, 256, 4, 0.01, "normal")
    q = make_query(rng, (1, 1, 64))
    return dict(dk=dk, dv=dv, xk=xk, xv=xv, q=q, K=4, klow=2, khigh=4,
                top_num=1, top_den=10, scale=1.0 / 8.0, atoms_k=ak,
                atoms_v=av, coefs_k=ck, coefs_v=cv)


# name -> (B, Hq, Hkv, T, seed)
DECODE_WORKLOADS = {
    "llama_layer_4k": (1, 32, 8, 4096, 1),
    "llama_layer_128k": (1, 32, 8, 131072, 3),
    "llama_layer_b8_32k": (8, 32, 8, 32768, 33),
}


def decode_case(name: str | None = None, *, B=None, Hq=None, Hkv=None, T=None,
                seed=None, n_atoms: int = 32768, d: int = 128, K: int = 16,
                klow: int = 3, khigh: int = 16, top_num: int = 1,
                top_den: int = 10, dk=None, dv=None) -> DecodeCase:
    """Llama-3.1-8B-shaped decode layer (or a custom shape).

    Draw order: Dk, Dv (skipped when given), key codes [B,Hkv,T,K],
    value codes, query [B,Hq,d].
    """
    if name is not None:
        B, Hq, Hkv, T, seed = DECODE_WORKLOADS[name]
    rng = np.random.default_rng(seed)
    if dk is None:
        dk = make_dictionary(rng, n_atoms, d, "bf16")
    if dv is None:
        dv = make_dictionary(rng, n_atoms, d, "bf16")
    n = B * Hkv * T
    kc = make_codes(rng, n, K, dk.shape[0]).reshape(B, Hkv, T, K)
    vc = make_codes(rng, n, K, dv.shape[0]).reshape(B, Hkv, T, K)
    q = make_query(rng, (B, Hq, d))
    return DecodeCase(name=name or f"custom_b{B}_h{Hq}_{Hkv}_t{T}", q=q,
                      dk=dk, dv=dv, key_codes=kc, val_codes=vc,
                      key_low=np.ascontiguousarray(kc[..., :klow]), K=K,
                      klow=klow, khigh=khigh, top_num=top_num,
                      top_den=top_den, scale=1.0 / math.sqrt(d))


def qwen_layer_case(layer: int, seed: int = 4, T: int = 262144) -> DecodeCase:
    """One layer of the Qwen-2.5-7B-shaped full-model decode step (28 query
    heads, 4 KV heads, head_dim 128, 262,144 coded tokens, batch 1), with
    that layer's own key/value dictionaries. Layer l uses seed
    seed*1000 + l; draw order as in `decode_case`."""
    return decode_case(B=1, Hq=28, Hkv=4, T=T, seed=seed * 1000 + layer)


def encode_case(n_tokens: int = 32768, n_heads: int = 8, seed: int = 2,
                stream: int = 0, n_atoms: int = 32768, d: int = 128,
                K: int = 16, n_vectors: int | None = None) -> EncodeCase:
    """Prefill-style encode workload for one stream (0 = keys, 1 = values):
    n_tokens * n_heads bf16 vectors, each a 16-atom combination with
    |N(0,1)| decreasing coefficients plus N(0, 0.05^2) noise, over that
    stream's 32,768-atom bf16 dictionary.

    Stream s uses seed*1000 + s. Draw order: dictionary, vectors.
    `n_vectors` draws only the first rows (same values as the full draw is
    NOT guaranteed; use it for standalone small cases).
    """
    rng = np.random.default_rng(seed * 1000 + stream)
    D = make_dictionary(rng, n_atoms, d, "bf16")
    n = n_vectors if n_vectors is not None else n_tokens * n_heads
    x, atoms, c = make_sparse_vectors(rng, D, n, K, 0.05, "absdesc")
    return EncodeCase(name=f"encode_s{stream}_n{n}", x=bf16_round(x),
                      dictionary=D, K=K, atoms=atoms, coefs=c)
