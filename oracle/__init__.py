"""fp64 CPU oracle for the dictionary-coded KV cache.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
NumPy statement of what the GPU library computes. Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import or call it; the
library itself never does and shares no code with it.

Sources (pages of "LLM Inference in a Flash!"):
  * review page, Summary: every key and value vector is kept as K=16 atoms
    of a 32,768-atom dictionary that is fixed per layer and per stream; the
    atoms are chosen greedily, one projection per step, without the
    least-squares re-solve of OMP; at decode time a Klow=3 score ranks all
    tokens and the best tenth is rescored with Khigh=16 atoms.
  * review page, Strengths (on replacing OMP for the hardware): the pursuit
    is greedy and never refits.
  * review page, FAQ (on the 15x compression figure): a vector is stored as
    16 atom indices plus coefficients; three atoms are enough to rank most
    tokens.
  * abstract page: keys and values are sums of fixed dictionary vectors.
  * review page, Summary and Strengths (integer-only execution): the
    integer softmax of integer_softmax.py.

Every function here has a pin in tests/test_oracle_*.py (closed forms,
invariants, brute force with exact rational arithmetic, hand-worked golden
fixtures); none is "parity unpinned". The readings taken where the pages are
silent are listed in each docstring.
"""
from .sdkv_oracle import (  # noqa: F401
    unpack_codes, pack_codes, mp_encode, omp_encode, decode_attn, select_topk,
    selected_count,
)
from .integer_softmax import int_softmax, int_exp_consts, INT_SOFTMAX_P_BITS  # noqa: F401
