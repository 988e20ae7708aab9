"""GPU parity of sdkv_decode_attn (through the C ABI) against the fp64 oracle,
stage by stage: U table, s_low, selected set, s_high, value weights, output.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def run_gpu(case, debug=True, key_low=True, ws=None, interleaved=False):
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    q = H.to_bf16(case.q)
    if case.dict_dtype == "bf16":
        dk, dv = H.to_bf16(case.dk), H.to_bf16(case.dv)
    else:
        dk, dv = H.to_f32(case.dk), H.to_f32(case.dv)
    if interleaved:
        # [B, Hkv, T, 2, K]: each token's key record, then its value record
        kc = H.to_words(np.stack([case.key_codes, case.val_codes], axis=3))
        vc = None
    else:
        kc, vc = H.to_words(case.key_codes), H.to_words(case.val_codes)
    kl = H.to_words(case.key_low) if key_low else None
    r = sd.sdkv_decode_attn(q, dk, dv, kc, vc, klow=case.klow, khigh=case.khigh,
                            top_num=case.top_num, top_den=case.top_den, scale=case.scale,
                            key_low=kl, debug=debug, workspace=ws)
    torch.cuda.synchronize()
    if not debug:
        return {"out": H.host(r)}
    return {k: H.host(v) for k, v in r.items()}


W_RTOL = H.W_RTOL


def compare(case, g, heads=None, w_tol=W_RTOL):
    """Oracle on the same inputs; full stage-by-stage comparison."""
    ref = oracle.decode_attn(case.q, case.dk, case.dv, case.key_codes, case.val_codes,
                             case.klow, case.khigh, case.top_num, case.top_den, case.scale)
    B, Hq = case.B, case.Hq
    m = ref["m"]
    rows = B * Hq
    u_err = H.rel_l2(g["u"], ref["u"])
    assert u_err < 1e-6, f"U table rel err {u_err}"
    sl_err = np.abs(g["s_low"].astype(np.float64) - ref["s_low"]).max()
    assert sl_err < 2e-6, f"s_low max abs err {sl_err}"
    sel = g["sel"].reshape(rows, m)
    ndiff = H.check_selection(sel, ref["s_low"].reshape(rows, -1), m)
    # s_high on the GPU's own selection, against the oracle's formula
    ref_g = ref if ndiff == 0 else oracle.decode_attn(
        case.q, case.dk, case.dv, case.key_codes, case.val_codes, case.klow, case.khigh,
        case.top_num, case.top_den, case.scale, sel=g["sel"])
    sh_err = np.abs(g["s_high"].astype(np.float64) - ref_g["s_high"]).max()
    assert sh_err < 5e-6, f"s_high max abs err {sh_err}"
    w_err = H.rel_l2(g["w"], ref_g["w"])
    assert w_err < w_tol, f"W rel err {w_err}"
    o_err = H.rel_l2(g["out"], ref["out"])
    assert o_err <= H.OUT_RTOL, f"output rel L2 {o_err}"
    o_err_g = H.rel_l2(g["out"], ref_g["out"])
    assert o_err_g <= H.OUT_RTOL
    H.log(f"  {case.name}: m={m} U {u_err:.2e} s_low {sl_err:.2e} sel-diff-rows {ndiff} "
          f"s_high {sh_err:.2e} W {w_err:.2e} out {o_err:.2e}")
    return ref


def tiny_decode_case():
    t = synth.tiny_case(0)
    ik, gk, _ = oracle.mp_encode(t["xk"], t["dk"], t["K"])
    iv, gv, _ = oracle.mp_encode(t["xv"], t["dv"], t["K"])
    kc = oracle.pack_codes(ik, gk).reshape(1, 1, 256, 4)
    vc = oracle.pack_codes(iv, gv).reshape(1, 1, 256, 4)
    return synth.DecodeCase(name="tiny", q=t["q"], dk=t["dk"], dv=t["dv"], key_codes=kc,
                            val_codes=vc, key_low=np.ascontiguousarray(kc[..., :2]), K=4,
                            klow=2, khigh=4, top_num=1, top_den=10, scale=1.0 / 8.0,
                            dict_dtype="f32")


def test_tiny_fp32_dictionaries():
    H.log("decode tiny (fp32 dictionaries, oracle-encoded codes)")
    case = tiny_decode_case()
    compare(case, run_gpu(case))


def test_llama_layer_4k():
    H.log("decode llama_layer_4k")
    case = synth.decode_case("llama_layer_4k")
    compare(case, run_gpu(case))


@pytest.mark.parametrize("T", [1, 9, 10, 11, 63, 64, 65, 513, 2049, 5000])
def test_ragged_context_lengths(T):
    H.log(f"decode ragged T={T}")
    case = synth.decode_case(B=1, Hq=4, Hkv=2, T=T, seed=100 + T, n_atoms=2048)
    compare(case, run_gpu(case))


def test_many_workgroups_per_row_and_batches():
    # T large enough that every row is split over several cooperating workgroups
    H.log("decode B=2 Hq=8 Hkv=2 T=40000")
    case = synth.decode_case(B=2, Hq=8, Hkv=2, T=40000, seed=7, n_atoms=4096)
    compare(case, run_gpu(case))


def test_cooperative_rows_with_the_selection_list_in_the_workspace():
    """128 rows of 20,000 tokens keeping the top half: each row is split over
    two workgroups of 16 keys per thread, and each workgroup selects ~5,000
    tokens, more than its LDS list holds, so the list and the rescored
    scores live in the workspace."""
    H.log("decode B=16 Hq=8 Hkv=2 T=20000 top 1/2")
    case = synth.decode_case(B=16, Hq=8, Hkv=2, T=20000, seed=15, n_atoms=1024, top_num=1,
                             top_den=2)
    compare(case, run_gpu(case))


def test_tall_value_weight_tiles_partly_filled():
    """40 query rows: the W.Dv kernel takes one 64-row tile, 24 rows of it
    empty, and merges the partials of 3 workgroups per row."""
    H.log("decode B=5 Hq=8 Hkv=2 T=9000 (40 rows)")
    case = synth.decode_case(B=5, Hq=8, Hkv=2, T=9000, seed=16, n_atoms=4096)
    compare(case, run_gpu(case))


@pytest.mark.parametrize("seed", range(20))
def test_random_shapes(seed):
    kw = H.random_decode_shape(seed)
    # record layouts in turn: a separate low plane, none (the first klow
    # words read from the key records), interleaved key/value records
    layout = seed % 3
    H.log(f"decode random shape {seed}, layout {layout}: {kw}")
    case = synth.decode_case(**kw)
    compare(case, run_gpu(case, key_low=layout == 0, interleaved=layout == 2))


def test_low_plane_from_key_codes():
    H.log("decode without a separate low plane")
    case = synth.decode_case(B=1, Hq=4, Hkv=1, T=3000, seed=8, n_atoms=1024)
    a = run_gpu(case, key_low=True)
    b = run_gpu(case, key_low=False)
    for k in ("u", "s_low", "sel", "s_high"):
        assert np.array_equal(a[k], b[k]), k
    compare(case, b)


def test_head_dim_64_and_K32():
    H.log("decode d=64, K=32, klow=5, khigh=20, top 1/4")
    case = synth.decode_case(B=1, Hq=6, Hkv=3, T=3001, seed=9, n_atoms=3000, d=64, K=32,
                             klow=5, khigh=20, top_num=1, top_den=4)
    compare(case, run_gpu(case))


def test_exact_ties_take_lowest_index():
    """Many tokens with identical key codes: identical scores; the selection
    must take the lowest token indices among the tied block."""
    H.log("decode constructed ties")
    case = synth.decode_case(B=1, Hq=2, Hkv=1, T=20000, seed=10, n_atoms=1024)
    kc = case.key_codes.copy()
    kc[0, 0, 5000:15000] = kc[0, 0, 123]   # 10,000 identical keys
    case.key_codes = kc
    case.key_low = np.ascontiguousarray(kc[..., :case.klow])
    g = run_gpu(case)
    ref = compare(case, g)
    assert np.array_equal(g["sel"].reshape(2, -1), ref["sel"].reshape(2, -1))


def test_deterministic_except_value_weights():
    case = synth.decode_case(B=1, Hq=8, Hkv=2, T=30000, seed=11, n_atoms=4096)
    a, b = run_gpu(case), run_gpu(case)
    for k in ("u", "s_low", "sel", "s_high"):
        assert np.array_equal(a[k], b[k]), k
    assert H.rel_l2(a["out"], b["out"]) < 1e-6


def test_llama_layer_128k_full_size():
    """The long-context workload at full size: 131,072 coded tokens, 32/8
    heads, 32,768-atom bf16 dictionaries, in the launch configuration the
    benchmark times."""
    H.log("decode llama_layer_128k (full size)")
    case = synth.decode_case("llama_layer_128k")
    g = run_gpu(case)
    compare(case, g)
    # the non-debug launch (as timed) gives the same output
    o = run_gpu(case, debug=False)["out"]
    assert H.rel_l2(o, g["out"]) < 1e-5


def test_llama_batch8_32k_full_size():
    H.log("decode llama_layer_b8_32k (full size)")
    case = synth.decode_case("llama_layer_b8_32k")
    compare(case, run_gpu(case))


@pytest.mark.slow
@pytest.mark.parametrize("layer", list(range(28)))
def test_qwen_full_model_layers(layer):
    """Every layer of the Qwen-2.5-7B-shaped full-model step (28 layers,
    28/4 heads, 262,144 tokens), each with its own key and value
    dictionaries, stage by stage against the oracle."""
    H.log(f"decode qwen layer {layer} (T=262144)")
    case = synth.qwen_layer_case(layer)
    compare(case, run_gpu(case))


def test_long_rows_many_workgroups():
    """262,144 tokens on the 32/8-head layer shape: each row is split over 16
    workgroups of 16 keys per thread, 512 workgroups in all (more than fit on
    the device at once), selection across workgroups with the one-barrier
    window select."""
    H.log("decode B=1 Hq=32 Hkv=8 T=262144")
    case = synth.decode_case(B=1, Hq=32, Hkv=8, T=262144, seed=12)
    compare(case, run_gpu(case))


def test_interleaved_key_value_records():
    """Key and value records side by side per token ([B, Hkv, T, 2, K], a
    record stride of 2K words): the same results as separate arrays, with and
    without a separate low plane, and against the oracle."""
    H.log("decode interleaved records B=2 Hq=8 Hkv=2 T=40000")
    case = synth.decode_case(B=2, Hq=8, Hkv=2, T=40000, seed=13, n_atoms=4096)
    a = run_gpu(case)
    for kl in (True, False):
        b = run_gpu(case, key_low=kl, interleaved=True)
        for k in ("u", "s_low", "sel", "s_high", "w", "out"):
            assert np.array_equal(a[k], b[k]), (kl, k)
    compare(case, b)


def test_interleaved_records_generic_path():
    """Interleaved records on the generic (K = 32, d = 64) path."""
    H.log("decode interleaved records d=64 K=32")
    case = synth.decode_case(B=1, Hq=6, Hkv=3, T=3001, seed=14, n_atoms=3000, d=64, K=32,
                             klow=5, khigh=20, top_num=1, top_den=4)
    a = run_gpu(case)
    b = run_gpu(case, interleaved=True)
    for k in ("u", "s_low", "sel", "s_high", "w", "out"):
        assert np.array_equal(a[k], b[k]), k
    compare(case, b)


def test_interleaved_records_128k_layer():
    """The benchmark's launch (non-debug, interleaved records) on the 128K
    layer equals the separate-array launch bit for bit."""
    H.log("decode llama_layer_128k interleaved vs separate (non-debug)")
    case = synth.decode_case("llama_layer_128k")
    a = run_gpu(case, debug=False)["out"]
    b = run_gpu(case, debug=False, interleaved=True)["out"]
    assert np.array_equal(a, b)
