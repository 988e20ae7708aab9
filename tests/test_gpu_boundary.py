"""GPU checks of the boundary's remaining contract through the C ABI: fp32
queries, the status word of a cross-workgroup wait that gives up, a whole
tiny case from GPU encode to GPU decode, and a decode step that appends the
new token's codes and then attends to them."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as H
from tests.test_gpu_decode import compare, run_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dict_dtype", ["bf16", "f32"])
def test_fp32_queries(dict_dtype):
    """fp32 queries (not bf16-representable) on bf16 and fp32 dictionaries,
    every stage against the oracle on the same fp32 query values."""
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    H.log(f"decode fp32 queries, {dict_dtype} dictionaries")
    case = synth.decode_case(B=2, Hq=8, Hkv=2, T=9000, seed=40, n_atoms=4096)
    rng = np.random.default_rng(41)
    case.q = rng.standard_normal(case.q.shape).astype(np.float32)
    assert not np.array_equal(case.q, synth.bf16_round(case.q))
    if dict_dtype == "f32":
        case.dk = synth.make_dictionary(rng, 4096, 128, "f32")
        case.dv = synth.make_dictionary(rng, 4096, 128, "f32")
        case.dict_dtype = "f32"
    dk = H.to_bf16(case.dk) if dict_dtype == "bf16" else H.to_f32(case.dk)
    dv = H.to_bf16(case.dv) if dict_dtype == "bf16" else H.to_f32(case.dv)
    r = sd.sdkv_decode_attn(H.to_f32(case.q), dk, dv, H.to_words(case.key_codes),
                            H.to_words(case.val_codes), klow=case.klow, khigh=case.khigh,
                            top_num=case.top_num, top_den=case.top_den, scale=case.scale,
                            key_low=H.to_words(case.key_low), debug=True)
    torch.cuda.synchronize()
    compare(case, {k: H.host(v) for k, v in r.items()})


def _forced_give_up(fn):
    import decode_attention_sparse_amd as sd
    sd.set_test_wait(64, 1)   # every wait gives up after 64 polls
    try:
        return fn()
    finally:
        sd.set_test_wait()


@pytest.mark.parametrize("flags", [{}, {"debug": True}, {"softmax": "int"},
                                   {"reading": "B"}, {"select": "kv"}])
def test_decode_wait_give_up_is_reported(flags):
    """Rows split over 20 workgroups; the host makes every cross-workgroup
    wait give up (a short poll limit and an arrival that never comes). The
    kernels still finish, the status word reads 1 and the binding raises
    SDKV_ERR_WAIT; the next normal call clears it and is correct."""
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    H.log(f"decode forced wait give-up {flags}")
    case = synth.decode_case(B=1, Hq=4, Hkv=2, T=40000, seed=42, n_atoms=2048)
    ws = sd.Workspace()
    args = (H.to_bf16(case.q), H.to_bf16(case.dk), H.to_bf16(case.dv),
            H.to_words(case.key_codes), H.to_words(case.val_codes))
    kw = dict(klow=case.klow, khigh=case.khigh, top_num=case.top_num, top_den=case.top_den,
              scale=case.scale, key_low=H.to_words(case.key_low), workspace=ws)

    def bad():
        with pytest.raises(sd.SdkvError) as e:
            sd.sdkv_decode_attn(*args, **kw, **flags)
        return e.value.status
    assert _forced_give_up(bad) == sd.SDKV_ERR_WAIT
    assert ws.status() == 1
    g = sd.sdkv_decode_attn(*args, **kw, debug=True)
    torch.cuda.synchronize()
    assert ws.status() == 0
    compare(case, {k: H.host(v) for k, v in g.items()})


def test_topk_wait_give_up_is_reported():
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    H.log("topk forced wait give-up")
    rng = np.random.default_rng(43)
    s = rng.standard_normal((2, 100000), dtype=np.float32)
    t = H.to_f32(s)
    ws = sd.Workspace()

    def bad():
        with pytest.raises(sd.SdkvError) as e:
            sd.sdkv_select_topk(t, 10000, workspace=ws)
        return e.value.status
    assert _forced_give_up(bad) == sd.SDKV_ERR_WAIT
    idx, _ = sd.sdkv_select_topk(t, 10000, workspace=ws)
    torch.cuda.synchronize()
    assert ws.status() == 0
    assert np.array_equal(H.host(idx), oracle.select_topk(s, 10000))


def test_tiny_case_gpu_encode_then_gpu_decode():
    """The tiny workload end to end on the GPU: keys and values encoded by
    sdkv_encode (fp32 dictionaries, K=4), those codes attended by
    sdkv_decode_attn (Klow=2, Khigh=4, top 10%, scale 1/8); against the
    oracle's encode followed by the oracle's decode."""
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    H.log("tiny case: GPU encode -> GPU decode vs oracle encode -> oracle decode")
    t = synth.tiny_case(0)
    dk, dv = H.to_f32(t["dk"]), H.to_f32(t["dv"])
    ck = sd.sdkv_encode(H.to_f32(t["xk"]), dk, 4)["codes"]
    cv = sd.sdkv_encode(H.to_f32(t["xv"]), dv, 4)["codes"]
    out = sd.sdkv_decode_attn(H.to_bf16(t["q"]), dk, dv, ck.reshape(1, 1, 256, 4),
                              cv.reshape(1, 1, 256, 4), klow=2, khigh=4, top_num=1,
                              top_den=10, scale=1.0 / 8.0)
    torch.cuda.synchronize()
    ik, gk, _ = oracle.mp_encode(t["xk"], t["dk"], 4)
    iv, gv, _ = oracle.mp_encode(t["xv"], t["dv"], 4)
    gik, _ = H.unpack_words(H.host(ck))
    giv, _ = H.unpack_words(H.host(cv))
    assert np.array_equal(gik, ik) and np.array_equal(giv, iv)
    kc = oracle.pack_codes(ik, gk).reshape(1, 1, 256, 4)
    vc = oracle.pack_codes(iv, gv).reshape(1, 1, 256, 4)
    ref = oracle.decode_attn(t["q"], t["dk"], t["dv"], kc, vc, 2, 4, 1, 10, 1.0 / 8.0)
    err = H.rel_l2(H.host(out), ref["out"])
    H.log(f"  tiny end to end: out rel L2 {err:.2e}")
    assert err <= H.OUT_RTOL


def test_append_then_attend():
    """One decode step: the new token's key and value vectors (8 KV heads)
    are encoded into slot T of a cache holding T = 4096 coded tokens
    (sdkv_append_tokens), then the step attends over all T + 1 tokens, with
    queries aimed at the new keys so that the new token is selected. The
    appended codes match the oracle's encode, and the output matches the
    oracle's decode over the cache as written."""
    import decode_attention_sparse_amd as sd
    torch = H.torch_mod()
    H.log("append at slot 4096, then attend over 4097 tokens")
    T = 4096
    case = synth.decode_case(B=1, Hq=32, Hkv=8, T=T + 1, seed=44)
    rng = np.random.default_rng(45)
    xk, _, _ = synth.make_sparse_vectors(rng, case.dk, 8, 16, 0.05, "absdesc")
    xv, _, _ = synth.make_sparse_vectors(rng, case.dv, 8, 16, 0.05, "absdesc")
    xk, xv = synth.bf16_round(xk), synth.bf16_round(xv)
    # queries: the new key of the head's KV group, plus noise
    q = np.repeat(xk, 4, axis=0)[None] * 3.0 + rng.standard_normal((1, 32, 128)).astype(np.float32)
    q = synth.bf16_round(q.astype(np.float32))
    kv = np.stack([case.key_codes, case.val_codes], axis=3)   # [1, 8, T+1, 2, 16]
    kv[:, :, T] = 0
    low = np.ascontiguousarray(case.key_low)
    low[:, :, T] = 0
    kv_t, low_t = H.to_words(kv), H.to_words(low)
    dk, dv = H.to_bf16(case.dk), H.to_bf16(case.dv)
    sd.sdkv_append_tokens(H.to_bf16(xk.reshape(1, 8, 128)), H.to_bf16(xv.reshape(1, 8, 128)),
                          dk, dv, kv_t, None, T, key_low=low_t)
    g = sd.sdkv_decode_attn(H.to_bf16(q), dk, dv, kv_t, None, klow=3, khigh=16, top_num=1,
                            top_den=10, scale=case.scale, key_low=low_t, debug=True)
    torch.cuda.synchronize()
    kvh = H.host(kv_t).view(np.uint32)
    lowh = H.host(low_t).view(np.uint32)
    # slots before T untouched, slot T holds the oracle's codes
    assert np.array_equal(kvh[:, :, :T], kv[:, :, :T])
    ik, gk, _ = oracle.mp_encode(xk, case.dk, 16)
    iv, gv, _ = oracle.mp_encode(xv, case.dv, 16)
    gi_k, gc_k = H.unpack_words(kvh[0, :, T, 0])
    gi_v, gc_v = H.unpack_words(kvh[0, :, T, 1])
    assert np.array_equal(gi_k, ik) and np.array_equal(gi_v, iv)
    assert np.all(np.abs(gc_k - gk) <= H.f16_half_ulp(gk) + H.COEF_TOL)
    assert np.array_equal(lowh[0, :, T], kvh[0, :, T, 0, :3])
    # the new token is selected by every head, and the output agrees
    sel = H.host(g["sel"]).reshape(32, -1)
    assert np.all(sel[:, -1] == T)
    written = synth.DecodeCase(name="appended", q=q, dk=case.dk, dv=case.dv,
                               key_codes=np.ascontiguousarray(kvh[:, :, :, 0]),
                               val_codes=np.ascontiguousarray(kvh[:, :, :, 1]),
                               key_low=np.ascontiguousarray(lowh), K=16, klow=3, khigh=16,
                               top_num=1, top_den=10, scale=case.scale)
    compare(written, {k: H.host(v) for k, v in g.items()})
