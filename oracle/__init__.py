"""fp64 CPU oracle for the dictionary-coded KV cache.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
NumPy statement of what the GPU library computes. Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import or call it; the
library itself never does and shares no code with it.

Sources (pages of "LLM Inference in a Flash!"):
  * review page, Summary: each key/value vector is a sparse combination of
    K=16 atoms of a per-layer, per-stream 32,768-atom dictionary, found by a
    projection-based greedy pursuit that replaces OMP so no least-squares
    refit is done; decode scores every token with Klow=3 atoms and refines
    the top 10% with Khigh=16.
  * review page, Strengths ("Hardware-aware replacement of OMP"): greedy,
    refit-free pursuit.
  * review page, FAQ ("What is the 15x KV cache compression"): vectors are
    stored as indices plus coefficients of 16 atoms; 3 atoms score most
    tokens.
  * abstract page: each KV vector is a linear combination of static
    dictionary vectors.

Every function here has a pin in tests/test_oracle_*.py (closed forms,
invariants, brute force with exact rational arithmetic, hand-worked golden
fixtures); none is "parity unpinned". The readings taken where the pages are
silent are listed in each docstring.
"""
from .sdkv_oracle import (  # noqa: F401
    unpack_codes, pack_codes, mp_encode, decode_attn, select_topk,
    selected_count,
)
