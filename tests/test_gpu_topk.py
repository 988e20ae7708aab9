"""GPU parity of sdkv_select_topk (through the C ABI): the selected index sets
are integer results and must equal the oracle exactly."""
import numpy as np
import pytest

import oracle
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def run(scores, k):
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    s = H.to_f32(scores)
    idx, thr = sd.sdkv_select_topk(s, k, thr_out=True)
    torch.cuda.synchronize()
    return H.host(idx), H.host(thr)


@pytest.mark.parametrize("rows,n,k,kind", [
    (1, 1, 1, "normal"), (1, 100, 10, "normal"), (3, 5000, 500, "ties"),
    (2, 100000, 10000, "normal"), (4, 70000, 1, "ties"), (2, 65537, 65537, "normal"),
    (5, 2047, 1024, "signed_zero"), (1, 1 << 22, 419431, "normal"), (300, 3000, 300, "ties"),
    # rows split over several workgroups at 32 keys per thread (P = 4 and 31)
    (64, 100000, 10000, "normal"), (16, 1000000, 100000, "ties"),
])
def test_topk_matches_oracle(rows, n, k, kind):
    H.log(f"topk rows={rows} n={n} k={k} {kind}")
    rng = np.random.default_rng(rows * 7 + n)
    if kind == "ties":
        s = rng.integers(-20, 20, (rows, n)).astype(np.float32)
    elif kind == "signed_zero":
        s = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], np.float32), (rows, n))
    else:
        s = rng.standard_normal((rows, n), dtype=np.float32)
    idx, thr = run(s, k)
    ref = oracle.select_topk(s, k)
    assert np.array_equal(idx, ref)
    for r in range(rows):
        assert thr[r] == np.sort(s[r].astype(np.float64))[::-1][k - 1]


def test_topk_strided_rows():
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    rng = np.random.default_rng(5)
    full = rng.standard_normal((6, 1200), dtype=np.float32)
    t = H.to_f32(full)[:, 100:1100]
    idx, _ = sd.sdkv_select_topk(t, 77)
    torch.cuda.synchronize()
    assert np.array_equal(H.host(idx), oracle.select_topk(full[:, 100:1100], 77))
