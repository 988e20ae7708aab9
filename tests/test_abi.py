"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/sdkv.h, and rejects bad arguments with the documented
status before anything is enqueued (so these calls never touch a device)."""
import ctypes
import re

import pytest

import decode_attention_sparse_amd as sd
import oracle

FAKE = 0x10000  # never dereferenced: every call below fails validation first


def declared_symbols():
    txt = open(sd.HEADER).read()
    return sorted(set(re.findall(r"SDKV_API\s+[\w\s\*]+?\b(sdkv_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = sd.lib()
    names = declared_symbols()
    assert len(names) == 13, names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.sdkv_abi_version() == 8


def test_status_strings():
    lib = sd.lib()
    for s in range(8):
        assert lib.sdkv_status_str(s) != b"unknown status"
    assert lib.sdkv_status_str(99) == b"unknown status"


def test_selected_count_matches_oracle():
    for T in (1, 2, 9, 10, 11, 63, 64, 65, 256, 4096, 131072, 262144):
        for num, den in ((1, 10), (1, 1), (3, 7), (1, 1000)):
            assert sd.selected_count(T, num, den) == oracle.selected_count(T, num, den)
    assert sd.selected_count(0, 1, 10) == 0
    assert sd.selected_count(10, 2, 1) == 0


def good_attn(**kw):
    a = sd.AttnArgs(q=FAKE, q_dtype=sd.SDKV_BF16, dk=FAKE, dv=FAKE, dict_dtype=sd.SDKV_BF16,
                    n_atoms=32768, B=1, Hq=32, Hkv=8, d=128, T=131072, key_low=FAKE,
                    key_codes=FAKE, val_codes=FAKE, K=16, klow=3, khigh=16, top_num=1,
                    top_den=10, scale=0.0883883, out=FAKE)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def ws_status(a):
    nb = ctypes.c_size_t(0)
    return sd.lib().sdkv_decode_attn_workspace(ctypes.byref(a), ctypes.byref(nb)), nb.value


def test_decode_workspace_query():
    st, nb = ws_status(good_attn())
    assert st == 0 and nb > 0
    st2, nb2 = ws_status(good_attn(T=4096))
    assert st2 == 0 and 0 < nb2 < nb
    assert ws_status(good_attn()) == (st, nb)


@pytest.mark.parametrize("field,value,status", [
    ("q", None, sd.SDKV_ERR_NULL), ("dk", None, sd.SDKV_ERR_NULL),
    ("dv", None, sd.SDKV_ERR_NULL), ("key_codes", None, sd.SDKV_ERR_NULL),
    ("val_codes", None, sd.SDKV_ERR_NULL), ("out", None, sd.SDKV_ERR_NULL),
    ("d", 96, sd.SDKV_ERR_SHAPE), ("T", 0, sd.SDKV_ERR_SHAPE),
    ("Hq", 30, sd.SDKV_ERR_SHAPE), ("B", 0, sd.SDKV_ERR_SHAPE),
    ("klow", 0, sd.SDKV_ERR_SHAPE), ("klow", 17, sd.SDKV_ERR_SHAPE),
    ("khigh", 17, sd.SDKV_ERR_SHAPE), ("K", 33, sd.SDKV_ERR_SHAPE),
    ("top_num", 0, sd.SDKV_ERR_SHAPE), ("top_num", 11, sd.SDKV_ERR_SHAPE),
    ("n_atoms", 70000, sd.SDKV_ERR_SHAPE), ("scale", float("inf"), sd.SDKV_ERR_SHAPE),
    ("q_dtype", 7, sd.SDKV_ERR_DTYPE), ("dict_dtype", -1, sd.SDKV_ERR_DTYPE),
    ("n_atoms", 40000, sd.SDKV_ERR_UNSUPPORTED),
    ("code_stride", 15, sd.SDKV_ERR_SHAPE), ("code_stride", -32, sd.SDKV_ERR_SHAPE),
    ("code_stride", 65537, sd.SDKV_ERR_SHAPE),
    ("softmax_mode", 2, sd.SDKV_ERR_SHAPE), ("softmax_mode", -1, sd.SDKV_ERR_SHAPE),
    ("select_mode", 2, sd.SDKV_ERR_SHAPE), ("select_mode", -1, sd.SDKV_ERR_SHAPE),
    ("reading", 2, sd.SDKV_ERR_SHAPE), ("reading", -1, sd.SDKV_ERR_SHAPE),
])
def test_decode_validation(field, value, status):
    a = good_attn(**{field: value})
    st, _ = ws_status(a)
    assert st == status
    # the compute entry point rejects it the same way, before any enqueue
    assert sd.lib().sdkv_decode_attn(ctypes.byref(a), ctypes.c_void_p(FAKE), 1 << 40, None) == status


def test_decode_code_stride_accepted():
    # dense (0), interleaved key/value records (2K) and any stride >= K plan the same workspace
    base = ws_status(good_attn())
    assert base[0] == sd.SDKV_OK
    for stride in (16, 32, 17, 65536):
        assert ws_status(good_attn(code_stride=stride)) == base


def test_decode_workspace_errors():
    a = good_attn()
    _, nb = ws_status(a)
    lib = sd.lib()
    assert lib.sdkv_decode_attn(ctypes.byref(a), None, nb, None) == sd.SDKV_ERR_NULL
    assert lib.sdkv_decode_attn(ctypes.byref(a), ctypes.c_void_p(FAKE), nb - 1, None) == sd.SDKV_ERR_WORKSPACE
    assert lib.sdkv_decode_attn(None, ctypes.c_void_p(FAKE), nb, None) == sd.SDKV_ERR_NULL
    assert lib.sdkv_decode_attn_workspace(ctypes.byref(a), None) == sd.SDKV_ERR_NULL


def good_enc(**kw):
    a = sd.EncodeArgs(x=FAKE, x_dtype=sd.SDKV_BF16, dict=FAKE, dict_dtype=sd.SDKV_BF16,
                      n=262144, d=128, n_atoms=32768, K=16, codes=FAKE)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("x", None, sd.SDKV_ERR_NULL), ("dict", None, sd.SDKV_ERR_NULL),
    ("codes", None, sd.SDKV_ERR_NULL), ("d", 32, sd.SDKV_ERR_SHAPE),
    ("n", 0, sd.SDKV_ERR_SHAPE), ("n_atoms", 65537, sd.SDKV_ERR_SHAPE),
    ("K", 0, sd.SDKV_ERR_SHAPE), ("K", 33, sd.SDKV_ERR_SHAPE),
    ("x_dtype", 5, sd.SDKV_ERR_DTYPE),
    ("codes_ld", 15, sd.SDKV_ERR_SHAPE), ("codes_ld", -1, sd.SDKV_ERR_SHAPE),
])
def test_encode_validation(field, value, status):
    a = good_enc(**{field: value})
    nb = ctypes.c_size_t(0)
    assert sd.lib().sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)) == status
    assert sd.lib().sdkv_encode(ctypes.byref(a), ctypes.c_void_p(FAKE), 1 << 40, None) == status


def test_encode_low_plane_klow_checked():
    a = good_enc(low_plane=FAKE, klow=0)
    nb = ctypes.c_size_t(0)
    assert sd.lib().sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)) == sd.SDKV_ERR_SHAPE
    a.klow = 3
    assert sd.lib().sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)) == 0 and nb.value > 0
    assert sd.lib().sdkv_encode(ctypes.byref(a), ctypes.c_void_p(FAKE), nb.value - 1, None) == sd.SDKV_ERR_WORKSPACE


def test_topk_validation():
    lib = sd.lib()
    nb = ctypes.c_size_t(0)
    assert lib.sdkv_select_topk_workspace(4, 1000, 100, ctypes.byref(nb)) == 0 and nb.value > 0
    assert lib.sdkv_select_topk_workspace(4, 1000, 1001, ctypes.byref(nb)) == sd.SDKV_ERR_SHAPE
    assert lib.sdkv_select_topk_workspace(0, 1000, 1, ctypes.byref(nb)) == sd.SDKV_ERR_SHAPE
    assert lib.sdkv_select_topk_workspace(1, 1 << 24, 1, ctypes.byref(nb)) == sd.SDKV_ERR_UNSUPPORTED
    V = ctypes.c_void_p
    assert lib.sdkv_select_topk(None, 4, 1000, 1000, 10, V(FAKE), None, V(FAKE), 1 << 30, None) == sd.SDKV_ERR_NULL
    assert lib.sdkv_select_topk(V(FAKE), 4, 1000, 999, 10, V(FAKE), None, V(FAKE), 1 << 30, None) == sd.SDKV_ERR_SHAPE
    assert lib.sdkv_select_topk(V(FAKE), 4, 1000, 1000, 10, V(FAKE), None, None, 1 << 30, None) == sd.SDKV_ERR_NULL
    assert lib.sdkv_select_topk(V(FAKE), 4, 1000, 1000, 10, V(FAKE), None, V(FAKE), 0, None) == sd.SDKV_ERR_WORKSPACE


def test_encode_strides_and_small_plan():
    nb = ctypes.c_size_t(0)
    lib = sd.lib()
    # a low-plane stride below klow is rejected; row strides >= the row are accepted
    a = good_enc(low_plane=FAKE, klow=3, low_ld=2)
    assert lib.sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)) == sd.SDKV_ERR_SHAPE
    a = good_enc(low_plane=FAKE, klow=3, low_ld=96, codes_ld=32 * 131072)
    assert lib.sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)) == 0
    # up to 64 vectors take the small path: two residual buffers plus two
    # winner tables of (n_atoms / 128) x n pairs, no dictionary copy
    for n in (1, 16, 64):
        a = good_enc(n=n)
        assert lib.sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)) == 0
        want = -(-2 * n * 128 * 4 // 256) * 256 + -(-2 * 256 * n * 8 // 256) * 256
        assert nb.value == want, (n, nb.value, want)
    a = good_enc(n=65)
    assert lib.sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)) == 0
    assert nb.value > 32768 * 128 * 2  # batch path: fp16 dictionary copy


def test_encode_pair_validation():
    lib = sd.lib()
    nb = ctypes.c_size_t(0)
    k, v = good_enc(n=8), good_enc(n=8)
    assert lib.sdkv_encode_pair_workspace(ctypes.byref(k), ctypes.byref(v), ctypes.byref(nb)) == 0
    one = ctypes.c_size_t(0)
    assert lib.sdkv_encode_workspace(ctypes.byref(k), ctypes.byref(one)) == 0
    assert nb.value == 2 * one.value  # both sides' scratch, each 256-byte aligned
    for field, value, status in (("n", 9, sd.SDKV_ERR_SHAPE), ("K", 8, sd.SDKV_ERR_SHAPE),
                                 ("n_atoms", 4096, sd.SDKV_ERR_SHAPE), ("d", 64, sd.SDKV_ERR_SHAPE),
                                 ("dict_dtype", sd.SDKV_F32, sd.SDKV_ERR_SHAPE),
                                 ("codes", None, sd.SDKV_ERR_NULL)):
        v2 = good_enc(n=8)
        setattr(v2, field, value)
        assert lib.sdkv_encode_pair_workspace(ctypes.byref(k), ctypes.byref(v2), ctypes.byref(nb)) == status
        assert lib.sdkv_encode_pair(ctypes.byref(k), ctypes.byref(v2), ctypes.c_void_p(FAKE), 1 << 30,
                                    None) == status
    big_k, big_v = good_enc(n=65), good_enc(n=65)
    assert lib.sdkv_encode_pair_workspace(ctypes.byref(big_k), ctypes.byref(big_v),
                                          ctypes.byref(nb)) == sd.SDKV_ERR_UNSUPPORTED
    k.x_dtype = sd.SDKV_F32  # input dtypes may differ
    assert lib.sdkv_encode_pair_workspace(ctypes.byref(k), ctypes.byref(v), ctypes.byref(nb)) == 0
    assert lib.sdkv_encode_pair(ctypes.byref(k), ctypes.byref(v), None, 1 << 30, None) == sd.SDKV_ERR_NULL
    assert lib.sdkv_encode_pair(ctypes.byref(k), ctypes.byref(v), ctypes.c_void_p(FAKE), nb.value - 1,
                                None) == sd.SDKV_ERR_WORKSPACE
    assert lib.sdkv_encode_pair_workspace(ctypes.byref(k), ctypes.byref(v), None) == sd.SDKV_ERR_NULL


def test_misaligned_pointers_rejected():
    lib = sd.lib()
    nb = ctypes.c_size_t(0)
    for field in ("x", "dict"):
        a = good_enc(**{field: FAKE + 8})
        assert lib.sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)) == sd.SDKV_ERR_UNSUPPORTED
    for field in ("q", "dk", "dv"):
        assert ws_status(good_attn(**{field: FAKE + 2}))[0] == sd.SDKV_ERR_UNSUPPORTED
    a = good_enc()
    assert lib.sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)) == 0
    assert lib.sdkv_encode(ctypes.byref(a), ctypes.c_void_p(FAKE + 4), nb.value, None) == sd.SDKV_ERR_UNSUPPORTED
    at = good_attn()
    _, anb = ws_status(at)
    assert lib.sdkv_decode_attn(ctypes.byref(at), ctypes.c_void_p(FAKE + 4), anb, None) == sd.SDKV_ERR_UNSUPPORTED


def test_decode_workspace_shared_selection():
    # the shared selection adds the group-summed U rows: B * Hkv * n_atoms floats
    st, nb = ws_status(good_attn())
    st2, nb2 = ws_status(good_attn(select_mode=sd.SDKV_SELECT_KV))
    assert st == st2 == 0 and nb2 - nb == 8 * 32768 * 4


def test_reading_b_needs_float_softmax():
    assert ws_status(good_attn(reading=sd.SDKV_READING_B))[0] == sd.SDKV_OK
    a = good_attn(reading=sd.SDKV_READING_B, softmax_mode=sd.SDKV_SOFTMAX_INT)
    assert ws_status(a)[0] == sd.SDKV_ERR_UNSUPPORTED


def test_omp_encoder_limits():
    nb = ctypes.c_size_t(0)
    lib = sd.lib()
    a = good_enc(n=16, algorithm=sd.SDKV_ENCODE_OMP)
    assert lib.sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)) == 0
    base = ctypes.c_size_t(0)
    b = good_enc(n=16)
    assert lib.sdkv_encode_workspace(ctypes.byref(b), ctypes.byref(base)) == 0
    # Q [n][K][d], R [n][K][K], z and the support [n][K]
    extra = 16 * 16 * (128 + 16 + 2) * 4
    assert nb.value == base.value + -(-extra // 256) * 256
    for field, value, status in (("n", 65, sd.SDKV_ERR_UNSUPPORTED),
                                 ("dict_dtype", sd.SDKV_F32, sd.SDKV_ERR_UNSUPPORTED),
                                 ("algorithm", 2, sd.SDKV_ERR_SHAPE)):
        c = good_enc(n=16, algorithm=sd.SDKV_ENCODE_OMP)
        setattr(c, field, value)
        assert lib.sdkv_encode_workspace(ctypes.byref(c), ctypes.byref(nb)) == status
    k, v = good_enc(n=8), good_enc(n=8, algorithm=sd.SDKV_ENCODE_OMP)
    assert lib.sdkv_encode_pair_workspace(ctypes.byref(k), ctypes.byref(v), ctypes.byref(nb)) == sd.SDKV_ERR_SHAPE


def test_fp32_queries_accepted():
    st, nb = ws_status(good_attn(q_dtype=sd.SDKV_F32))
    assert st == 0 and nb > 0


def test_status_word_is_workspace_word_zero():
    """The status word the header documents is word 0 of the workspace, and
    the binding turns a nonzero word into SdkvError(SDKV_ERR_WAIT). Checked
    on a host-memory stand-in for a workspace (no kernel runs here)."""
    import torch
    txt = open(sd.HEADER).read()
    assert "Word 0 (uint32) of the workspace" in txt
    assert re.search(r"#define SDKV_ERR_WAIT 7\b", txt)
    ws = sd.Workspace(device="cpu")
    assert ws.status() == 0
    ws.buf = torch.zeros(256, dtype=torch.uint8)
    ws.check()
    ws.buf[0] = 1
    assert ws.status() == 1
    with pytest.raises(sd.SdkvError) as e:
        ws.check("probe")
    assert e.value.status == sd.SDKV_ERR_WAIT
    assert b"gave up" in sd.lib().sdkv_status_str(sd.SDKV_ERR_WAIT)
    ws.buf[0] = 0
    ws.buf[3] = 1
    assert ws.status() == 1 << 24


def test_temporary_workspace_kept_for_the_launch_stream(monkeypatch):
    """A workspace the binding makes for one call is returned to the caller
    (kept alive across the C call) and tied to a non-current launch stream
    with record_stream, so the caching allocator cannot hand its memory to
    other work before that stream has finished with it."""
    recorded = []

    class FakeBuf:
        def __init__(self, n):
            self.n = n

        def numel(self):
            return self.n

        def data_ptr(self):
            return 4096

        def record_stream(self, st):
            recorded.append(st)

    class FakeStream:
        pass

    class FakeCuda:
        @staticmethod
        def current_stream():
            return "current"

    class FakeTorch:
        cuda = FakeCuda

    monkeypatch.setattr(sd.Workspace, "get", lambda self, n: FakeBuf(n))
    monkeypatch.setattr(sd, "_torch", lambda: FakeTorch)
    other = FakeStream()
    ws, ptr, n = sd._ws(None, 1000, other)
    assert isinstance(ws, sd.Workspace) and ptr == 4096 and n == 1000
    assert recorded == [other]
    ws2, _, _ = sd._ws(None, 1000, "current")
    assert recorded == [other]
    mine = sd.Workspace()
    ws3, _, _ = sd._ws(mine, 1000, other)
    assert ws3 is mine and recorded == [other]
