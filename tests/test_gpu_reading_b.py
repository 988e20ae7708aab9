"""GPU parity of reading B (SDKV_READING_B: every token enters the softmax,
the unselected ones with their s_low and first Klow value pairs) through the
C ABI, against the oracle's reading="B": scores, selection, value weights and
output, with the value low words from a separate plane or from the value
records (dense and interleaved layouts), alone and with the shared
selection."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

W_RTOL = H.W_RTOL    # fixed-point sums handed over as binary16


def run(case, *, val_low=True, interleaved=False, select="head", debug=True, reading="B",
        top=None):
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    q = H.to_bf16(case.q)
    dk, dv = H.to_bf16(case.dk), H.to_bf16(case.dv)
    if interleaved:
        kc = H.to_words(np.stack([case.key_codes, case.val_codes], axis=3))
        vc = None
    else:
        kc, vc = H.to_words(case.key_codes), H.to_words(case.val_codes)
    vl = H.to_words(np.ascontiguousarray(case.val_codes[..., :case.klow])) if val_low else None
    tn, td = top if top else (case.top_num, case.top_den)
    r = sd.sdkv_decode_attn(q, dk, dv, kc, vc, klow=case.klow, khigh=case.khigh, top_num=tn,
                            top_den=td, scale=case.scale, key_low=H.to_words(case.key_low),
                            debug=debug, select=select, reading=reading, val_low=vl)
    torch.cuda.synchronize()
    if not debug:
        return {"out": H.host(r)}
    return {k: H.host(v) for k, v in r.items()}


def oracle_run(case, **kw):
    return oracle.decode_attn(case.q, case.dk, case.dv, case.key_codes, case.val_codes,
                              case.klow, case.khigh, case.top_num, case.top_den, case.scale, **kw)


def check(case, g, label, select="head"):
    ref = oracle_run(case, reading="B", select=select)
    m = ref["m"]
    rows = case.B * case.Hq
    sl_err = np.abs(g["s_low"].astype(np.float64) - ref["s_low"]).max()
    assert sl_err < 1e-5, f"{label}: s_low max abs err {sl_err}"
    ndiff = H.check_selection(g["sel"].reshape(rows, m), ref["s_low"].reshape(rows, -1), m)
    ref_g = ref if ndiff == 0 else oracle_run(case, reading="B", select=select, sel=g["sel"])
    sh_err = np.abs(g["s_high"].astype(np.float64) - ref_g["s_high"]).max()
    assert sh_err < 5e-6, f"{label}: s_high max abs err {sh_err}"
    w_err = H.rel_l2(g["w"], ref_g["w"])
    assert w_err < W_RTOL, f"{label}: W rel err {w_err}"
    o_err = H.rel_l2(g["out"], ref["out"])
    assert o_err <= H.OUT_RTOL, f"{label}: output rel L2 {o_err}"
    ref_a = oracle_run(case, select=select)
    d_ab = H.rel_l2(ref["out"], ref_a["out"])
    H.log(f"  {label}: m={m} s_low {sl_err:.2e} sel-diff-rows {ndiff} s_high {sh_err:.2e} "
          f"W {w_err:.2e} out {o_err:.2e} (readings A and B differ by {d_ab:.2e})")


def test_reading_b_llama_layer_4k():
    H.log("reading B: llama_layer_4k (value low plane)")
    case = synth.decode_case("llama_layer_4k")
    check(case, run(case), "llama 4k")


@pytest.mark.parametrize("T", [1, 11, 513, 5000])
def test_reading_b_ragged_from_value_records(T):
    H.log(f"reading B: ragged T={T}, value words from the records")
    case = synth.decode_case(B=1, Hq=4, Hkv=2, T=T, seed=500 + T, n_atoms=2048)
    check(case, run(case, val_low=False), f"T={T}")


@pytest.mark.parametrize("val_low", [True, False])
def test_reading_b_rows_over_many_workgroups(val_low):
    H.log(f"reading B: B=2 Hq=8 Hkv=2 T=40000, interleaved records, value plane {val_low}")
    case = synth.decode_case(B=2, Hq=8, Hkv=2, T=40000, seed=37, n_atoms=4096)
    check(case, run(case, val_low=val_low, interleaved=True), f"T=40000 plane={val_low}")


def test_reading_b_with_shared_selection():
    H.log("reading B + shared selection: B=1 Hq=8 Hkv=2 T=20000")
    case = synth.decode_case(B=1, Hq=8, Hkv=2, T=20000, seed=38, n_atoms=4096)
    check(case, run(case, select="kv"), "B + shared", select="kv")


def test_reading_b_selection_list_in_the_workspace():
    H.log("reading B: B=16 Hq=8 Hkv=2 T=20000 top 1/2 (selection list in the workspace)")
    case = synth.decode_case(B=16, Hq=8, Hkv=2, T=20000, seed=41, n_atoms=1024, top_num=1,
                             top_den=2)
    check(case, run(case, val_low=False), "top 1/2")


def test_reading_b_at_full_selection_equals_reading_a():
    H.log("reading B with every token selected")
    case = synth.decode_case(B=1, Hq=4, Hkv=2, T=3000, seed=39, n_atoms=2048)
    a = run(case, reading="A", top=(1, 1))
    b = run(case, top=(1, 1))
    for key in ("s_low", "sel", "s_high"):
        assert np.array_equal(a[key], b[key]), key
    assert H.rel_l2(b["out"], a["out"]) < 1e-5


def test_reading_b_128k_layer():
    """The 128K layer in reading B with a value low plane, as the benchmark
    launches it: one KV group against the oracle run on that group alone,
    and the non-debug launch."""
    H.log("reading B: llama_layer_128k")
    case = synth.decode_case("llama_layer_128k")
    g = run(case, interleaved=True)
    G = case.Hq // case.Hkv
    gk = 6
    sub = synth.decode_case(B=1, Hq=G, Hkv=1, T=case.T, seed=0, n_atoms=64, dk=case.dk,
                            dv=case.dv)
    sub.q = case.q[:, gk * G:(gk + 1) * G].copy()
    sub.key_codes = case.key_codes[:, gk:gk + 1].copy()
    sub.val_codes = case.val_codes[:, gk:gk + 1].copy()
    ref = oracle_run(sub, reading="B")
    hs = slice(gk * G, (gk + 1) * G)
    ndiff = H.check_selection(g["sel"][0, hs], ref["s_low"][0], ref["m"])
    o_err = H.rel_l2(g["out"][:, hs], ref["out"])
    assert o_err <= H.OUT_RTOL, o_err
    o = run(case, interleaved=True, debug=False)["out"]
    assert H.rel_l2(o, g["out"]) < 1e-5
    H.log(f"  128k reading B: group {gk} sel-diff-rows {ndiff} out {o_err:.2e}")


@pytest.mark.parametrize("seed", range(8))
def test_reading_b_random_shapes(seed):
    kw = H.random_decode_shape(seed, base=9200)
    # value low words in turn from their own plane, the value records, the
    # interleaved records
    layout = seed % 3
    H.log(f"reading B: random shape {seed}, layout {layout}: {kw}")
    case = synth.decode_case(**kw)
    check(case, run(case, val_low=layout == 0, interleaved=layout == 2), f"random {seed}")
