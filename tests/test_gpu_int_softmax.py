"""GPU parity of the integer-only softmax (SDKV_SOFTMAX_INT) through the C ABI:
the integer probabilities bit for bit against the oracle's integer steps on
the GPU's own fp32 scores, the value weights and output on those, the output
against the oracle's own integer-mode run, and the distance to the fp32
softmax (the quantization effect, bounded by the oracle pins)."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

P1 = 2.0 ** oracle.INT_SOFTMAX_P_BITS
W_RTOL = H.W_RTOL    # fixed-point sums handed over as binary16
QUANT_RTOL = 2e-2   # integer vs fp32 softmax, output rel-L2


def run_int(case, *, interleaved=False, debug=True, softmax="int"):
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    q = H.to_bf16(case.q)
    dk, dv = H.to_bf16(case.dk), H.to_bf16(case.dv)
    if interleaved:
        kc = H.to_words(np.stack([case.key_codes, case.val_codes], axis=3))
        vc = None
    else:
        kc, vc = H.to_words(case.key_codes), H.to_words(case.val_codes)
    r = sd.sdkv_decode_attn(q, dk, dv, kc, vc, klow=case.klow, khigh=case.khigh,
                            top_num=case.top_num, top_den=case.top_den, scale=case.scale,
                            key_low=H.to_words(case.key_low), debug=debug, softmax=softmax)
    torch.cuda.synchronize()
    if not debug:
        return {"out": H.host(r)}
    return {k: H.host(v) for k, v in r.items()}


def oracle_run(case, **kw):
    return oracle.decode_attn(case.q, case.dk, case.dv, case.key_codes, case.val_codes,
                              case.klow, case.khigh, case.top_num, case.top_den, case.scale, **kw)


def check(case, g, label):
    m = oracle.selected_count(case.T, case.top_num, case.top_den)
    # integer steps, bit for bit, on the GPU's selection and fp32 scores
    ref_g = oracle_run(case, sel=g["sel"], softmax="int", s_high_in=g["s_high"])
    assert np.array_equal(g["p_int"], ref_g["p_int"]), \
        f"{label}: {int((g['p_int'] != ref_g['p_int']).sum())} of {g['p_int'].size} p differ"
    assert np.all(np.abs(g["p_int"].astype(np.int64).sum(axis=-1) - P1) <= m + 2)
    w_err = H.rel_l2(g["w"], ref_g["w"])
    assert w_err < W_RTOL, f"{label}: W rel err {w_err}"
    o_g = H.rel_l2(g["out"], ref_g["out"])
    assert o_g <= 1e-3, f"{label}: out rel err on the GPU's p {o_g}"
    # against the oracle's own integer-mode run (its selection and scores)
    ref = oracle_run(case, softmax="int")
    o_err = H.rel_l2(g["out"], ref["out"])
    assert o_err <= H.OUT_RTOL, f"{label}: output rel L2 {o_err}"
    # distance to the fp32 softmax
    ref_f = oracle_run(case)
    q_err = H.rel_l2(g["out"], ref_f["out"])
    assert q_err <= QUANT_RTOL, f"{label}: integer vs float softmax {q_err}"
    H.log(f"  {label}: m={m} p_int exact, W {w_err:.2e}, out {o_err:.2e} "
          f"(on GPU p {o_g:.2e}), vs fp32 softmax {q_err:.2e}")


def test_int_softmax_llama_layer_4k():
    H.log("integer softmax: llama_layer_4k")
    case = synth.decode_case("llama_layer_4k")
    check(case, run_int(case), "llama 4k")


@pytest.mark.parametrize("T", [1, 2, 11, 513, 5000])
def test_int_softmax_ragged(T):
    H.log(f"integer softmax: ragged T={T}")
    case = synth.decode_case(B=1, Hq=4, Hkv=2, T=T, seed=300 + T, n_atoms=2048)
    check(case, run_int(case), f"T={T}")


def test_int_softmax_rows_over_many_workgroups():
    # every row split over several workgroups: both exchanges are used
    H.log("integer softmax: B=2 Hq=8 Hkv=2 T=40000 (interleaved records)")
    case = synth.decode_case(B=2, Hq=8, Hkv=2, T=40000, seed=17, n_atoms=4096)
    check(case, run_int(case, interleaved=True), "T=40000")


def test_int_softmax_selection_list_in_the_workspace():
    # ~5,000 selected tokens per workgroup: the integer exponentials are
    # stored over the scores in the workspace list
    H.log("integer softmax: B=16 Hq=8 Hkv=2 T=20000 top 1/2")
    case = synth.decode_case(B=16, Hq=8, Hkv=2, T=20000, seed=19, n_atoms=1024, top_num=1,
                             top_den=2)
    check(case, run_int(case), "top 1/2")


def test_int_softmax_zero_query_uniform():
    """q = 0: every score is 0 (k = 30), so within each row every selected
    token gets the same integer probability."""
    H.log("integer softmax: zero query")
    case = synth.decode_case(B=1, Hq=4, Hkv=2, T=3000, seed=21, n_atoms=1024)
    case.q[...] = 0.0
    g = run_int(case)
    p = g["p_int"].reshape(4, -1)
    assert np.all(p == p[:, :1])
    check(case, g, "zero query")


def test_int_softmax_128k_layer_sampled():
    """The 128K layer in integer mode, as the benchmark launches it: p_int bit
    for bit on every head (integer steps on the GPU's scores), the output of
    one KV group against the oracle run on that group alone, and the
    non-debug launch."""
    H.log("integer softmax: llama_layer_128k")
    case = synth.decode_case("llama_layer_128k")
    g = run_int(case, interleaved=True)
    B, Hq, Hkv = case.B, case.Hq, case.Hkv
    G = Hq // Hkv
    for h in range(Hq):
        p = oracle.int_softmax(g["s_high"][0, h])
        assert np.array_equal(g["p_int"][0, h], p), f"head {h}"
    gk = 3
    sub = synth.decode_case(B=1, Hq=G, Hkv=1, T=case.T, seed=0, n_atoms=64, dk=case.dk,
                            dv=case.dv)
    sub.q = case.q[:, gk * G:(gk + 1) * G].copy()
    sub.key_codes = case.key_codes[:, gk:gk + 1].copy()
    sub.val_codes = case.val_codes[:, gk:gk + 1].copy()
    ref = oracle_run(sub, softmax="int")
    o_err = H.rel_l2(g["out"][:, gk * G:(gk + 1) * G], ref["out"])
    assert o_err <= H.OUT_RTOL, o_err
    o = run_int(case, interleaved=True, debug=False)["out"]
    assert H.rel_l2(o, g["out"]) < 1e-5
    H.log(f"  128k: p_int exact on {Hq} heads; group {gk} out {o_err:.2e}")


@pytest.mark.parametrize("seed", range(8))
def test_int_softmax_random_shapes(seed):
    kw = H.random_decode_shape(seed, base=9100)
    H.log(f"integer softmax: random shape {seed}: {kw}")
    case = synth.decode_case(**kw)
    check(case, run_int(case, interleaved=seed % 2 == 1), f"random {seed}")
