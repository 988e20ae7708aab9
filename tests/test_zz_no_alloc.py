"""The allocation-free append encode (sdkv_encode_pair_noalloc, static
per-GPU scratch) against sdkv_encode_pair with a caller workspace, through
the C ABI: identical outputs bit for bit, on consecutive calls whose second
is smaller (the scratch keeps the previous call's contents)."""
import ctypes

import numpy as np
import pytest

import synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def make_side(torch, sd, x, D, K, klow, omp):
    n, d = x.shape
    out = dict(codes=torch.full((n, K), -1, dtype=torch.int32, device="cuda"),
               coef=torch.full((n, K), float("nan"), dtype=torch.float32, device="cuda"),
               rn=torch.full((n,), float("nan"), dtype=torch.float32, device="cuda"),
               low=torch.full((n, klow), -1, dtype=torch.int32, device="cuda"))
    a = sd.EncodeArgs(x=x.data_ptr(), x_dtype=sd.SDKV_BF16, dict=D.data_ptr(),
                      dict_dtype=sd.SDKV_BF16, n=n, d=d, n_atoms=D.shape[0], K=K,
                      codes=out["codes"].data_ptr(), coef_f32=out["coef"].data_ptr(),
                      resid_norm=out["rn"].data_ptr(), low_plane=out["low"].data_ptr(),
                      klow=klow, algorithm=sd.SDKV_ENCODE_OMP if omp else sd.SDKV_ENCODE_PURSUIT)
    return a, out


def one_case(n, N, K, klow, omp, seed):
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    rng = np.random.default_rng(seed)
    Dk = synth.make_dictionary(rng, N, 128, "bf16")
    Dv = synth.make_dictionary(rng, N, 128, "bf16")
    xk, _, _ = synth.make_sparse_vectors(rng, Dk, n, 16, 0.05, "absdesc")
    xv, _, _ = synth.make_sparse_vectors(rng, Dv, n, 16, 0.05, "absdesc")
    t = dict(xk=H.to_bf16(synth.bf16_round(xk)), xv=H.to_bf16(synth.bf16_round(xv)),
             Dk=H.to_bf16(Dk), Dv=H.to_bf16(Dv))
    res = []
    for noalloc in (False, True):
        ak, ok = make_side(torch, sd, t["xk"], t["Dk"], K, klow, omp)
        av, ov = make_side(torch, sd, t["xv"], t["Dv"], K, klow, omp)
        if noalloc:
            st = sd.lib().sdkv_encode_pair_noalloc(ctypes.byref(ak), ctypes.byref(av), None)
            assert st == sd.SDKV_OK, st
        else:
            sd.sdkv_encode_pair(ak, av)
        torch.cuda.synchronize()
        res.append({**{"k_" + k: H.host(v) for k, v in ok.items()},
                    **{"v_" + k: H.host(v) for k, v in ov.items()}})
    ref, got = res
    for k in ref:
        assert np.array_equal(ref[k].view(np.uint8), got[k].view(np.uint8)), k
    H.log(f"  noalloc n={n} N={N} K={K} omp={omp}: identical to the workspace call")


def test_noalloc_pair_matches_workspace_pair_on_consecutive_calls():
    H.log("noalloc append encode: 16 vectors, then 5, then an OMP pair of 8")
    one_case(16, 32768, 16, 3, False, 70)
    one_case(5, 4096, 8, 2, False, 71)
    one_case(8, 2048, 12, 3, True, 72)
