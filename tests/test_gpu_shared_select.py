"""GPU parity of the selection shared by the query heads of a KV head
(SDKV_SELECT_KV) through the C ABI, against the oracle's select="kv": the
shared ranking score, the selected set (identical except tokens tied with
the threshold), the per-head rescore, value weights and output; and the
reductions the mode must satisfy (one head per group equals per-head
selection; every head of a group takes the same set)."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

W_RTOL = H.W_RTOL    # fixed-point sums handed over as binary16


def run(case, *, select="kv", softmax="float", interleaved=False, debug=True, q_f32=False):
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    q = H.to_f32(case.q) if q_f32 else H.to_bf16(case.q)
    if case.dict_dtype == "f32":
        dk, dv = H.to_f32(case.dk), H.to_f32(case.dv)
    else:
        dk, dv = H.to_bf16(case.dk), H.to_bf16(case.dv)
    if interleaved:
        kc = H.to_words(np.stack([case.key_codes, case.val_codes], axis=3))
        vc = None
    else:
        kc, vc = H.to_words(case.key_codes), H.to_words(case.val_codes)
    r = sd.sdkv_decode_attn(q, dk, dv, kc, vc, klow=case.klow, khigh=case.khigh,
                            top_num=case.top_num, top_den=case.top_den, scale=case.scale,
                            key_low=H.to_words(case.key_low), debug=debug, softmax=softmax,
                            select=select)
    torch.cuda.synchronize()
    if not debug:
        return {"out": H.host(r)}
    return {k: H.host(v) for k, v in r.items()}


def oracle_run(case, **kw):
    return oracle.decode_attn(case.q, case.dk, case.dv, case.key_codes, case.val_codes,
                              case.klow, case.khigh, case.top_num, case.top_den, case.scale, **kw)


def check(case, g, label, softmax="float"):
    B, Hq, Hkv = case.B, case.Hq, case.Hkv
    G = Hq // Hkv
    ref = oracle_run(case, select="kv", softmax=softmax)
    m = ref["m"]
    rows = B * Hq
    sl_err = np.abs(g["s_low"].astype(np.float64) - ref["s_low"]).max()
    assert sl_err < 1e-5, f"{label}: shared score max abs err {sl_err}"
    sel = g["sel"].reshape(B, Hkv, G, m)
    assert np.all(sel == sel[:, :, :1]), f"{label}: heads of a group selected differently"
    ndiff = H.check_selection(g["sel"].reshape(rows, m), ref["s_low"].reshape(rows, -1), m)
    ref_g = ref if ndiff == 0 else oracle_run(case, select="kv", softmax=softmax, sel=g["sel"])
    sh_err = np.abs(g["s_high"].astype(np.float64) - ref_g["s_high"]).max()
    assert sh_err < 5e-6, f"{label}: s_high max abs err {sh_err}"
    w_err = H.rel_l2(g["w"], ref_g["w"])
    assert w_err < W_RTOL, f"{label}: W rel err {w_err}"
    o_err = H.rel_l2(g["out"], ref["out"])
    assert o_err <= H.OUT_RTOL, f"{label}: output rel L2 {o_err}"
    H.log(f"  {label}: m={m} shared score {sl_err:.2e} sel-diff-rows {ndiff} s_high {sh_err:.2e} "
          f"W {w_err:.2e} out {o_err:.2e}")


def test_shared_select_llama_layer_4k():
    H.log("shared selection: llama_layer_4k")
    case = synth.decode_case("llama_layer_4k")
    check(case, run(case), "llama 4k")


@pytest.mark.parametrize("T", [1, 11, 513, 5000])
def test_shared_select_ragged(T):
    H.log(f"shared selection: ragged T={T}")
    case = synth.decode_case(B=2, Hq=6, Hkv=2, T=T, seed=400 + T, n_atoms=2048)
    check(case, run(case), f"T={T}")


def test_shared_select_rows_over_many_workgroups():
    H.log("shared selection: B=2 Hq=8 Hkv=2 T=40000 (interleaved records)")
    case = synth.decode_case(B=2, Hq=8, Hkv=2, T=40000, seed=27, n_atoms=4096)
    check(case, run(case, interleaved=True), "T=40000")


def test_shared_select_selection_list_in_the_workspace():
    H.log("shared selection: B=16 Hq=8 Hkv=2 T=20000 top 1/2 (selection list in the workspace)")
    case = synth.decode_case(B=16, Hq=8, Hkv=2, T=20000, seed=30, n_atoms=1024, top_num=1,
                             top_den=2)
    check(case, run(case), "top 1/2")


def test_shared_select_with_integer_softmax():
    H.log("shared selection + integer softmax: B=1 Hq=8 Hkv=2 T=20000")
    case = synth.decode_case(B=1, Hq=8, Hkv=2, T=20000, seed=28, n_atoms=4096)
    g = run(case, softmax="int")
    check(case, g, "shared + int", softmax="int")
    ref_g = oracle_run(case, select="kv", softmax="int", sel=g["sel"], s_high_in=g["s_high"])
    assert np.array_equal(g["p_int"], ref_g["p_int"])


def test_one_head_per_group_equals_per_head_selection():
    H.log("shared selection with G = 1")
    case = synth.decode_case(B=1, Hq=4, Hkv=4, T=9000, seed=29, n_atoms=2048)
    a = run(case, select="head")
    k = run(case, select="kv")
    for key in ("s_low", "sel", "s_high", "out"):
        assert np.array_equal(a[key], k[key]), key


def test_shared_select_128k_layer():
    """The 128K layer as launched by the benchmark, with the shared selection:
    every group's heads agree, one group is checked against the oracle run on
    that group alone, and the non-debug launch gives the same output."""
    H.log("shared selection: llama_layer_128k")
    case = synth.decode_case("llama_layer_128k")
    g = run(case, interleaved=True)
    G = case.Hq // case.Hkv
    m = g["sel"].shape[-1]
    sel = g["sel"].reshape(case.B, case.Hkv, G, m)
    assert np.all(sel == sel[:, :, :1])
    gk = 5
    sub = synth.decode_case(B=1, Hq=G, Hkv=1, T=case.T, seed=0, n_atoms=64, dk=case.dk,
                            dv=case.dv)
    sub.q = case.q[:, gk * G:(gk + 1) * G].copy()
    sub.key_codes = case.key_codes[:, gk:gk + 1].copy()
    sub.val_codes = case.val_codes[:, gk:gk + 1].copy()
    ref = oracle_run(sub, select="kv")
    hs = slice(gk * G, (gk + 1) * G)
    ndiff = H.check_selection(g["sel"][0, hs], ref["s_low"][0], m)
    o_err = H.rel_l2(g["out"][:, hs], ref["out"])
    assert o_err <= H.OUT_RTOL, o_err
    o = run(case, interleaved=True, debug=False)["out"]
    assert H.rel_l2(o, g["out"]) < 1e-5
    H.log(f"  128k shared: group {gk} sel-diff-rows {ndiff} out {o_err:.2e}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (28, 4)])
def test_shared_select_fp32_queries(Hq, Hkv):
    """fp32 queries (not bf16-representable): the group rows of the ranking
    table come from the fp32 sum of each group's query rows (G = 4 and 7)."""
    H.log(f"shared selection: fp32 queries, Hq={Hq} Hkv={Hkv}")
    case = synth.decode_case(B=1, Hq=Hq, Hkv=Hkv, T=9000, seed=450 + Hq, n_atoms=4096)
    rng = np.random.default_rng(451 + Hq)
    case.q = rng.standard_normal(case.q.shape).astype(np.float32)
    assert not np.array_equal(case.q, synth.bf16_round(case.q))
    check(case, run(case, q_f32=True), f"fp32 q, G={Hq // Hkv}")


def test_shared_select_many_groups():
    """80 KV-head groups (B=10, Hkv=8): the U-table kernel stages their summed
    queries in two passes of 64."""
    H.log("shared selection: B=10 Hq=16 Hkv=8 T=3000 (80 groups)")
    case = synth.decode_case(B=10, Hq=16, Hkv=8, T=3000, seed=460, n_atoms=2048)
    check(case, run(case), "80 groups")


def test_shared_select_fp32_dictionary():
    """fp32 dictionaries: the group rows of U are summed from the heads' U rows
    by their own kernel."""
    H.log("shared selection: fp32 dictionaries, B=2 Hq=8 Hkv=2 T=5000")
    case = synth.decode_case(B=2, Hq=8, Hkv=2, T=5000, seed=470, n_atoms=2048)
    rng = np.random.default_rng(471)
    case.dk = synth.make_dictionary(rng, 2048, 128, "f32")
    case.dv = synth.make_dictionary(rng, 2048, 128, "f32")
    case.dict_dtype = "f32"
    check(case, run(case), "fp32 dictionaries")


@pytest.mark.parametrize("seed", range(8))
def test_shared_select_random_shapes(seed):
    kw = H.random_decode_shape(seed, base=9300)
    H.log(f"shared selection: random shape {seed}: {kw}")
    case = synth.decode_case(**kw)
    check(case, run(case, interleaved=seed % 2 == 1, q_f32=seed % 4 == 2), f"random {seed}")
