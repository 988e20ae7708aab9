"""Python binding of libsdkv (dictionary-coded KV cache on MI355X).

Argument marshalling only: every computation runs in the HIP kernels of
libsdkv.so, reached through its C ABI (include/sdkv.h). PyTorch supplies
device memory and the current HIP stream. Importing works without a GPU;
calling a compute entry point needs the built library and a GPU, and raises
if either is missing (there is no CPU fallback).

Entry points (same names as the C ABI):
  sdkv_encode(x, dictionary, K, ...)        greedy pursuit codes
  sdkv_decode_attn(q, dk, dv, key_codes, val_codes, ...)
  sdkv_select_topk(scores, k, ...)
Code words are carried in torch.int32 tensors holding the uint32 bit
patterns (atom index in bits 0-15, binary16 coefficient in bits 16-31).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsdkv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "sdkv.h")

SDKV_OK, SDKV_ERR_NULL, SDKV_ERR_SHAPE, SDKV_ERR_DTYPE = 0, 1, 2, 3
SDKV_ERR_UNSUPPORTED, SDKV_ERR_WORKSPACE, SDKV_ERR_DEVICE, SDKV_ERR_WAIT = 4, 5, 6, 7
ABI_VERSION = 8
SDKV_BF16, SDKV_F32 = 0, 1
SDKV_SOFTMAX_FLOAT, SDKV_SOFTMAX_INT = 0, 1
_SOFTMAX = {"float": SDKV_SOFTMAX_FLOAT, "int": SDKV_SOFTMAX_INT}
SDKV_SELECT_HEAD, SDKV_SELECT_KV = 0, 1
_SELECT = {"head": SDKV_SELECT_HEAD, "kv": SDKV_SELECT_KV}
SDKV_READING_A, SDKV_READING_B = 0, 1
SDKV_ENCODE_PURSUIT, SDKV_ENCODE_OMP = 0, 1
_ALGORITHM = {"pursuit": SDKV_ENCODE_PURSUIT, "omp": SDKV_ENCODE_OMP}
_READING = {"A": SDKV_READING_A, "B": SDKV_READING_B}

c_void_p, c_int32, c_int64, c_float = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
c_size_t = ctypes.c_size_t


class EncodeArgs(ctypes.Structure):
    _fields_ = [("x", c_void_p), ("x_dtype", c_int32), ("dict", c_void_p),
                ("dict_dtype", c_int32), ("n", c_int64), ("d", c_int32),
                ("n_atoms", c_int32), ("K", c_int32), ("codes", c_void_p),
                ("codes_ld", c_int64), ("coef_f32", c_void_p), ("resid_norm", c_void_p),
                ("low_plane", c_void_p), ("low_ld", c_int64), ("klow", c_int32),
                ("stage_events", c_void_p), ("algorithm", c_int32)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("q_dtype", c_int32), ("dk", c_void_p),
                ("dv", c_void_p), ("dict_dtype", c_int32), ("n_atoms", c_int32),
                ("B", c_int32), ("Hq", c_int32), ("Hkv", c_int32), ("d", c_int32),
                ("T", c_int64), ("key_low", c_void_p), ("key_codes", c_void_p),
                ("val_codes", c_void_p), ("code_stride", c_int64), ("K", c_int32), ("klow", c_int32),
                ("khigh", c_int32), ("top_num", c_int64), ("top_den", c_int64),
                ("scale", c_float), ("out", c_void_p), ("u", c_void_p),
                ("s_low", c_void_p), ("sel", c_void_p), ("s_high", c_void_p),
                ("w", c_void_p), ("stage_events", c_void_p), ("softmax_mode", c_int32),
                ("p_int", c_void_p), ("select_mode", c_int32), ("reading", c_int32),
                ("val_low", c_void_p)]


class SdkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib().sdkv_status_str(status).decode() if _LIB else str(status)
        super().__init__(f"{where}: status {status} ({msg})")


_LIB = None


def _lib():
    """Load libsdkv.so from the package directory (built by
    `python -m decode_attention_sparse_amd.build`)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m decode_attention_sparse_amd.build`")
        # Load torch's HIP runtime first so that libsdkv binds to the same
        # runtime instance (both carry the soname libamdhip64.so.7); streams
        # and events from torch are then valid handles inside the library.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        lib.sdkv_abi_version.restype = c_int32
        if lib.sdkv_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI {lib.sdkv_abi_version()}, the binding "
                              f"expects {ABI_VERSION}: rebuild it")
        lib.sdkv_test_set_wait.restype = None
        lib.sdkv_test_set_wait.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        lib.sdkv_status_str.restype = ctypes.c_char_p
        lib.sdkv_status_str.argtypes = [c_int32]
        lib.sdkv_selected_count.restype = c_int64
        lib.sdkv_selected_count.argtypes = [c_int64, c_int64, c_int64]
        lib.sdkv_encode_workspace.restype = c_int32
        lib.sdkv_encode_workspace.argtypes = [P(EncodeArgs), P(c_size_t)]
        lib.sdkv_encode.restype = c_int32
        lib.sdkv_encode.argtypes = [P(EncodeArgs), c_void_p, c_size_t, c_void_p]
        lib.sdkv_encode_pair_workspace.restype = c_int32
        lib.sdkv_encode_pair_workspace.argtypes = [P(EncodeArgs), P(EncodeArgs), P(c_size_t)]
        lib.sdkv_encode_pair.restype = c_int32
        lib.sdkv_encode_pair.argtypes = [P(EncodeArgs), P(EncodeArgs), c_void_p, c_size_t, c_void_p]
        lib.sdkv_encode_pair_noalloc.restype = c_int32
        lib.sdkv_encode_pair_noalloc.argtypes = [P(EncodeArgs), P(EncodeArgs), c_void_p]
        lib.sdkv_decode_attn_workspace.restype = c_int32
        lib.sdkv_decode_attn_workspace.argtypes = [P(AttnArgs), P(c_size_t)]
        lib.sdkv_decode_attn.restype = c_int32
        lib.sdkv_decode_attn.argtypes = [P(AttnArgs), c_void_p, c_size_t, c_void_p]
        lib.sdkv_select_topk_workspace.restype = c_int32
        lib.sdkv_select_topk_workspace.argtypes = [c_int64, c_int64, c_int64, P(c_size_t)]
        lib.sdkv_select_topk.restype = c_int32
        lib.sdkv_select_topk.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_int64,
                                         c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        _LIB = lib
    return _LIB


def lib():
    return _lib()


def set_test_wait(polls: int = 0, extra: int = 0):
    """Test hook (sdkv_test_set_wait): later calls' cross-workgroup waits give
    up after `polls` polls and wait for `extra` arrivals that never come;
    set_test_wait() restores the normal bounds."""
    _lib().sdkv_test_set_wait(polls, extra)


def _check(status: int, where: str):
    if status != SDKV_OK:
        raise SdkvError(status, where)


# ---------------------------------------------------------------------------
# torch marshalling helpers
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SDKV_BF16
    if t.dtype == torch.float32:
        return SDKV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class Workspace:
    """A reusable device workspace (a uint8 torch tensor that grows on demand).

    Word 0 of a decode-attention or top-k workspace is the call's status word
    (include/sdkv.h): status() reads it (synchronising) and check() raises
    SdkvError(SDKV_ERR_WAIT) when a cross-workgroup wait gave up."""

    def __init__(self, device=None):
        self.buf = None
        self.device = device

    def get(self, nbytes: int):
        torch = _torch()
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device or "cuda")
        return self.buf

    def status(self) -> int:
        """The status word (uint32 at byte 0) after the last call's work has
        completed (a device-to-host copy, which waits for it)."""
        if self.buf is None:
            return 0
        b = self.buf[:4].cpu().tolist()
        return b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24)

    def check(self, where: str = "status word"):
        if self.status() != 0:
            raise SdkvError(SDKV_ERR_WAIT, where)


def _ws(workspace, nbytes, stream=None):
    """(workspace, pointer, size). The caller keeps the returned Workspace
    referenced until the call has been enqueued; a workspace made here for
    one call is also tied to the launch stream, so the caching allocator
    does not hand its memory out again before that stream's work is done."""
    own = workspace is None
    if own:
        workspace = Workspace()
    buf = workspace.get(nbytes)
    if own and stream is not None:
        torch = _torch()
        if stream != torch.cuda.current_stream():
            buf.record_stream(stream)
    return workspace, buf.data_ptr(), buf.numel()


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------
def selected_count(T: int, top_num: int, top_den: int) -> int:
    return int(_lib().sdkv_selected_count(T, top_num, top_den))


def _events(stage_events):
    """ctypes array of hipEvent_t handles (ints), or None."""
    if stage_events is None:
        return None, None
    arr = (c_void_p * len(stage_events))(*[int(e) for e in stage_events])
    return arr, ctypes.cast(arr, c_void_p).value


def sdkv_encode(x, dictionary, K: int, *, codes=None, coef_f32=None, resid_norm=None,
                low_plane=None, klow: int = 0, workspace: Optional[Workspace] = None,
                stream=None, stage_events=None, algorithm: str = "pursuit"):
    """Greedy-pursuit codes of the rows of x [n, d] over `dictionary`
    [n_atoms, d] (bf16 or fp32 GPU tensors). Output tensors are allocated
    when not given: codes int32 [n, K]; pass coef_f32=True / resid_norm=True /
    low_plane=True (with klow) to request the optional outputs.
    algorithm="omp" takes the OMP comparison encoder (SDKV_ENCODE_OMP)."""
    torch = _torch()
    n, d = x.shape
    dev = x.device
    if codes is None:
        codes = torch.empty((n, K), dtype=torch.int32, device=dev)
    if coef_f32 is True:
        coef_f32 = torch.empty((n, K), dtype=torch.float32, device=dev)
    if resid_norm is True:
        resid_norm = torch.empty((n,), dtype=torch.float32, device=dev)
    if low_plane is True:
        low_plane = torch.empty((n, klow), dtype=torch.int32, device=dev)
    a = EncodeArgs(x=_dev(x, "x"), x_dtype=_dtype_code(x), dict=_dev(dictionary, "dictionary"),
                   dict_dtype=_dtype_code(dictionary), n=n, d=d, n_atoms=dictionary.shape[0],
                   K=K, codes=_dev(codes, "codes"),
                   coef_f32=_dev(coef_f32 if coef_f32 is not False else None, "coef_f32"),
                   resid_norm=_dev(resid_norm if resid_norm is not False else None, "resid_norm"),
                   low_plane=_dev(low_plane if low_plane is not False else None, "low_plane"),
                   klow=klow, algorithm=_ALGORITHM[algorithm])
    ev_keep, a.stage_events = _events(stage_events)
    nb = c_size_t(0)
    _check(_lib().sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)), "sdkv_encode_workspace")
    ws, wp, wn = _ws(workspace, nb.value, stream)
    _check(_lib().sdkv_encode(ctypes.byref(a), ctypes.c_void_p(wp), wn, _stream(stream)),
           "sdkv_encode")
    del ws
    res = {"codes": codes}
    if coef_f32 is not None and coef_f32 is not False:
        res["coef_f32"] = coef_f32
    if resid_norm is not None and resid_norm is not False:
        res["resid_norm"] = resid_norm
    if low_plane is not None and low_plane is not False:
        res["low_plane"] = low_plane
    return res


def attn_args(q, dk, dv, key_codes, val_codes, klow, khigh, top_num, top_den, scale, out,
              key_low=None, u=None, s_low=None, sel=None, s_high=None, w=None,
              softmax: str = "float", p_int=None, select: str = "head", reading: str = "A",
              val_low=None) -> AttnArgs:
    B, Hq, d = q.shape
    if val_codes is None:
        # one tensor [B, Hkv, T, 2, K]: each token's key record, then its value record
        if key_codes.dim() != 5 or key_codes.shape[3] != 2:
            raise ValueError("with val_codes=None, key_codes must be [B, Hkv, T, 2, K]")
        _, Hkv, T, _, K = key_codes.shape
        kp = _dev(key_codes, "key_codes")
        vp, stride = kp + 4 * K, 2 * K
    else:
        _, Hkv, T, K = key_codes.shape
        kp, vp, stride = _dev(key_codes, "key_codes"), _dev(val_codes, "val_codes"), 0
    return AttnArgs(q=_dev(q, "q"), q_dtype=_dtype_code(q), dk=_dev(dk, "dk"), dv=_dev(dv, "dv"),
                    dict_dtype=_dtype_code(dk), n_atoms=dk.shape[0], B=B, Hq=Hq, Hkv=Hkv, d=d,
                    T=T, key_low=_dev(key_low, "key_low"), key_codes=kp,
                    val_codes=vp, code_stride=stride, K=K, klow=klow, khigh=khigh,
                    top_num=top_num, top_den=top_den, scale=scale, out=_dev(out, "out"),
                    u=_dev(u, "u"), s_low=_dev(s_low, "s_low"), sel=_dev(sel, "sel"),
                    s_high=_dev(s_high, "s_high"), w=_dev(w, "w"),
                    softmax_mode=_SOFTMAX[softmax], p_int=_dev(p_int, "p_int"),
                    select_mode=_SELECT[select], reading=_READING[reading],
                    val_low=_dev(val_low, "val_low"))


def decode_attn_workspace_bytes(args: AttnArgs) -> int:
    nb = c_size_t(0)
    _check(_lib().sdkv_decode_attn_workspace(ctypes.byref(args), ctypes.byref(nb)),
           "sdkv_decode_attn_workspace")
    return nb.value


def sdkv_decode_attn(q, dk, dv, key_codes, val_codes, *, klow: int, khigh: int,
                     top_num: int = 1, top_den: int = 10, scale: Optional[float] = None,
                     key_low=None, out=None, debug: bool = False, softmax: str = "float",
                     select: str = "head", reading: str = "A", val_low=None,
                     workspace: Optional[Workspace] = None, stream=None, stage_events=None,
                     check: bool = True):
    """Hierarchical coded decode attention. q [B,Hq,d] bf16; dk, dv
    [n_atoms,d] bf16/fp32; key_codes, val_codes int32 [B,Hkv,T,K], or
    key_codes int32 [B,Hkv,T,2,K] (each token's key record, then its value
    record) with val_codes=None; optional key_low int32 [B,Hkv,T,klow].
    softmax="int" takes the integer-only softmax (SDKV_SOFTMAX_INT);
    select="kv" shares each KV head's selection among its query heads
    (SDKV_SELECT_KV); reading="B" lets every token into the softmax
    (SDKV_READING_B), with val_low int32 [B,Hkv,T,klow] the first klow
    value words (optional). q may be bf16 or fp32.
    With check=True (the default) the call waits for its work and raises
    SdkvError(SDKV_ERR_WAIT) if the workspace's status word reports that a
    cross-workgroup wait gave up.
    Returns out fp32 [B,Hq,d], or with debug=True a dict that also holds u,
    s_low, sel, s_high and w (and p_int in integer mode)."""
    torch = _torch()
    B, Hq, d = q.shape
    T = key_codes.shape[2]
    dev = q.device
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    dbg = {}
    if debug:
        m = selected_count(T, top_num, top_den)
        N = dk.shape[0]
        dbg = dict(u=torch.empty((B, Hq, N), dtype=torch.float32, device=dev),
                   s_low=torch.empty((B, Hq, T), dtype=torch.float32, device=dev),
                   sel=torch.empty((B, Hq, m), dtype=torch.int32, device=dev),
                   s_high=torch.empty((B, Hq, m), dtype=torch.float32, device=dev),
                   w=torch.empty((B, Hq, N), dtype=torch.float32, device=dev))
        if softmax == "int":
            dbg["p_int"] = torch.empty((B, Hq, m), dtype=torch.int32, device=dev)
    a = attn_args(q, dk, dv, key_codes, val_codes, klow, khigh, top_num, top_den, scale, out,
                  key_low=key_low, softmax=softmax, select=select, reading=reading,
                  val_low=val_low, **dbg)
    ev_keep, a.stage_events = _events(stage_events)
    ws, wp, wn = _ws(workspace, decode_attn_workspace_bytes(a), stream)
    _check(_lib().sdkv_decode_attn(ctypes.byref(a), ctypes.c_void_p(wp), wn, _stream(stream)),
           "sdkv_decode_attn")
    if check:
        ws.check("sdkv_decode_attn")
    if debug:
        dbg["out"] = out
        return dbg
    return out


def _encode_rows_args(x, dictionary, K, codes_ptr, codes_ld, low_ptr, low_ld, klow):
    """EncodeArgs writing code rows at codes_ptr + i * codes_ld words (and
    low-plane rows at low_ptr + i * low_ld), for appends into a cache."""
    n, d = x.shape
    return EncodeArgs(x=_dev(x, "x"), x_dtype=_dtype_code(x), dict=_dev(dictionary, "dictionary"),
                      dict_dtype=_dtype_code(dictionary), n=n, d=d, n_atoms=dictionary.shape[0],
                      K=K, codes=codes_ptr, codes_ld=codes_ld, low_plane=low_ptr, low_ld=low_ld,
                      klow=klow if low_ptr else 0)


def _encode_into(a, workspace, stream):
    nb = c_size_t(0)
    _check(_lib().sdkv_encode_workspace(ctypes.byref(a), ctypes.byref(nb)), "sdkv_encode_workspace")
    ws, wp, wn = _ws(workspace, nb.value, stream)
    _check(_lib().sdkv_encode(ctypes.byref(a), ctypes.c_void_p(wp), wn, _stream(stream)),
           "sdkv_encode")
    del ws


def sdkv_encode_pair(ak: "EncodeArgs", av: "EncodeArgs", workspace: Optional[Workspace] = None,
                     stream=None):
    """Two small encodes (n <= 64, same shape) in one sequence of launches,
    from marshalled EncodeArgs; each side gets what sdkv_encode gives it."""
    nb = c_size_t(0)
    _check(_lib().sdkv_encode_pair_workspace(ctypes.byref(ak), ctypes.byref(av), ctypes.byref(nb)),
           "sdkv_encode_pair_workspace")
    ws, wp, wn = _ws(workspace, nb.value, stream)
    _check(_lib().sdkv_encode_pair(ctypes.byref(ak), ctypes.byref(av), ctypes.c_void_p(wp), wn,
                                   _stream(stream)), "sdkv_encode_pair")
    del ws


def sdkv_encode_pair_noalloc(ak: "EncodeArgs", av: "EncodeArgs", stream=None):
    """sdkv_encode_pair with the library's static per-GPU scratch instead of
    a workspace: nothing is allocated (see include/sdkv.h)."""
    _check(_lib().sdkv_encode_pair_noalloc(ctypes.byref(ak), ctypes.byref(av), _stream(stream)),
           "sdkv_encode_pair_noalloc")


def sdkv_append_tokens(xk, xv, dk, dv, key_codes, val_codes, t: int, *, key_low=None,
                       workspace: Optional[Workspace] = None, stream=None):
    """Encode one decode step's new key and value vectors xk, xv [B, Hkv, d]
    and write their codes into slot t of the cache, in place: key_codes and
    val_codes int32 [B, Hkv, T, K], or key_codes [B, Hkv, T, 2, K] with
    val_codes=None (records side by side); key_low int32 [B, Hkv, T, klow]
    receives the key's first klow words. With n = B*Hkv <= 64 both sides
    take the fp32-accurate small-batch path together, in one sequence of K + 1
    launches (sdkv_encode_pair); larger batches make two sdkv_encode calls."""
    B, Hkv, d = xk.shape
    if val_codes is None:
        if key_codes.dim() != 5 or key_codes.shape[3] != 2:
            raise ValueError("with val_codes=None, key_codes must be [B, Hkv, T, 2, K]")
        T, K = key_codes.shape[2], key_codes.shape[4]
        base = _dev(key_codes, "key_codes")
        stride = 2 * K
        kp, vp = base + 4 * t * stride, base + 4 * (t * stride + K)
    else:
        T, K = key_codes.shape[2], key_codes.shape[3]
        stride = K
        kp = _dev(key_codes, "key_codes") + 4 * t * K
        vp = _dev(val_codes, "val_codes") + 4 * t * K
    if not 0 <= t < T:
        raise ValueError(f"slot {t} outside the cache's {T} tokens")
    if tuple(key_codes.shape[:2]) != (B, Hkv) or tuple(xv.shape) != (B, Hkv, d):
        raise ValueError("cache and new-token shapes disagree")
    lp, lld, klow = 0, 0, 0
    if key_low is not None:
        klow = key_low.shape[3]
        lp = _dev(key_low, "key_low") + 4 * t * klow
        lld = T * klow
    ws = workspace if workspace is not None else Workspace()
    ak = _encode_rows_args(xk.reshape(B * Hkv, d), dk, K, kp, T * stride, lp, lld, klow)
    av = _encode_rows_args(xv.reshape(B * Hkv, d), dv, K, vp, T * stride, 0, 0, 0)
    if B * Hkv <= 64 and dk.shape == dv.shape and dk.dtype == dv.dtype:
        sdkv_encode_pair(ak, av, ws, stream)
    else:
        _encode_into(ak, ws, stream)
        _encode_into(av, ws, stream)


class DecodeCall:
    """A decode-attention call whose arguments and workspace are marshalled
    once; launch() then costs one C call. Keeps references to every tensor it
    points at. Same arguments as sdkv_decode_attn (without debug outputs)."""

    def __init__(self, q, dk, dv, key_codes, val_codes, *, klow: int, khigh: int,
                 top_num: int = 1, top_den: int = 10, scale: Optional[float] = None,
                 key_low=None, out=None, softmax: str = "float", select: str = "head",
                 reading: str = "A", val_low=None,
                 workspace: Optional[Workspace] = None, stream=None):
        torch = _torch()
        B, Hq, d = q.shape
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        self.out = out
        self._keep = (q, dk, dv, key_codes, val_codes, key_low, val_low, out)
        self.args = attn_args(q, dk, dv, key_codes, val_codes, klow, khigh, top_num, top_den,
                              scale, out, key_low=key_low, softmax=softmax, select=select,
                              reading=reading, val_low=val_low)
        self.ws = workspace if workspace is not None else Workspace()
        _, wp, wn = _ws(self.ws, decode_attn_workspace_bytes(self.args))
        self._wsp, self._wsn = ctypes.c_void_p(wp), wn
        self._stream = _stream(stream)
        self._argp = ctypes.byref(self.args)
        self._fn = _lib().sdkv_decode_attn
        self._ev = None

    def launch(self, stage_events=None):
        if stage_events is not None:
            self._ev, self.args.stage_events = _events(stage_events)
        else:
            self.args.stage_events = None
        st = self._fn(self._argp, self._wsp, self._wsn, self._stream)
        if st != SDKV_OK:
            raise SdkvError(st, "sdkv_decode_attn")
        return self.out

    def check(self):
        """Raise SdkvError(SDKV_ERR_WAIT) if the last launch's status word
        reports a wait that gave up (waits for the launch to complete)."""
        self.ws.check("sdkv_decode_attn")


class EncodeCall:
    """An encode call marshalled once (see DecodeCall); codes int32 [n, K]."""

    def __init__(self, x, dictionary, K: int, *, codes=None, resid_norm=None,
                 workspace: Optional[Workspace] = None, stream=None):
        torch = _torch()
        n, d = x.shape
        if codes is None:
            codes = torch.empty((n, K), dtype=torch.int32, device=x.device)
        self.codes, self.resid_norm = codes, resid_norm
        self._keep = (x, dictionary, codes, resid_norm)
        self.args = EncodeArgs(x=_dev(x, "x"), x_dtype=_dtype_code(x),
                               dict=_dev(dictionary, "dictionary"),
                               dict_dtype=_dtype_code(dictionary), n=n, d=d,
                               n_atoms=dictionary.shape[0], K=K, codes=_dev(codes, "codes"),
                               coef_f32=None, resid_norm=_dev(resid_norm, "resid_norm"),
                               low_plane=None, klow=0)
        nb = c_size_t(0)
        _check(_lib().sdkv_encode_workspace(ctypes.byref(self.args), ctypes.byref(nb)),
               "sdkv_encode_workspace")
        self.ws = workspace if workspace is not None else Workspace()
        _, wp, wn = _ws(self.ws, nb.value)
        self._wsp, self._wsn = ctypes.c_void_p(wp), wn
        self._stream = _stream(stream)
        self._argp = ctypes.byref(self.args)
        self._fn = _lib().sdkv_encode
        self._ev = None

    def launch(self, stage_events=None):
        if stage_events is not None:
            self._ev, self.args.stage_events = _events(stage_events)
        else:
            self.args.stage_events = None
        st = self._fn(self._argp, self._wsp, self._wsn, self._stream)
        if st != SDKV_OK:
            raise SdkvError(st, "sdkv_encode")
        return self.codes


def sdkv_select_topk(scores, k: int, *, idx_out=None, thr_out=None,
                     workspace: Optional[Workspace] = None, stream=None, check: bool = True):
    """Indices (int32, ascending) of the k largest entries of each row of the
    fp32 GPU tensor `scores` [rows, n] (rows may be strided: row stride =
    scores.stride(0)); ties to the lower index. Returns (idx, thr). With
    check=True the call waits for its work and raises on a status word that
    reports a wait that gave up (see sdkv_decode_attn)."""
    torch = _torch()
    if scores.dim() == 1:
        scores = scores[None]
    rows, n = scores.shape
    if scores.dtype != torch.float32 or not scores.is_cuda or scores.stride(1) != 1:
        raise ValueError("scores must be a GPU float32 tensor with unit column stride")
    ld = scores.stride(0) if rows > 1 else n
    if idx_out is None:
        idx_out = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    if thr_out is True:
        thr_out = torch.empty((rows,), dtype=torch.float32, device=scores.device)
    nb = c_size_t(0)
    _check(_lib().sdkv_select_topk_workspace(rows, n, k, ctypes.byref(nb)),
           "sdkv_select_topk_workspace")
    ws, wp, wn = _ws(workspace, nb.value, stream)
    thr_ptr = thr_out.data_ptr() if thr_out is not None and thr_out is not False else None
    _check(_lib().sdkv_select_topk(ctypes.c_void_p(scores.data_ptr()), rows, n, ld, k,
                                   ctypes.c_void_p(_dev(idx_out, "idx_out")),
                                   ctypes.c_void_p(thr_ptr), ctypes.c_void_p(wp), wn,
                                   _stream(stream)), "sdkv_select_topk")
    if check:
        ws.check("sdkv_select_topk")
    return idx_out, (thr_out if thr_ptr else None)


__all__ = ["sdkv_encode", "sdkv_decode_attn", "sdkv_select_topk", "selected_count",
           "SDKV_SOFTMAX_FLOAT", "SDKV_SOFTMAX_INT", "SDKV_SELECT_HEAD", "SDKV_SELECT_KV",
           "SDKV_READING_A", "SDKV_READING_B", "SDKV_ENCODE_PURSUIT", "SDKV_ENCODE_OMP",
           "Workspace", "SdkvError", "lib", "LIB_PATH", "HEADER", "EncodeArgs", "AttnArgs",
           "SDKV_ERR_WAIT", "set_test_wait",
           "sdkv_append_tokens", "sdkv_encode_pair", "sdkv_encode_pair_noalloc",
           "attn_args", "decode_attn_workspace_bytes", "DecodeCall", "EncodeCall"]
