"""ctypes binding over librfw_atf.so (include/atf.h), same names as the C ABI.

Argument marshalling only: tensors become device pointers, torch's current
HIP stream becomes the call's stream, and torch allocates the caller-owned
workspace.  Every step of the computation runs in the library's HIP kernels;
there is no fallback of any kind -- if the library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librfw_atf.so")

ATF_OK, ATF_ERR_INVALID_ARG, ATF_ERR_UNSUPPORTED, ATF_ERR_WORKSPACE, ATF_ERR_HIP = range(5)
ATF_F32, ATF_BF16 = 0, 1
W_INF = np.iinfo(np.int64).max

# every symbol include/atf.h declares
EXPORTED = (
    "atf_status_string", "atf_version", "atf_window_table", "atf_skipped_pair_products",
    "atf_prefill_workspace_bytes", "atf_prefill", "atf_prefill_prepare_kv",
    "atf_prefill_attend", "atf_prefill_chunk", "atf_prefill_chunk_workspace_bytes",
    "atf_prefill_cache_bytes", "atf_prefill_cache_append", "atf_prefill_cached_scratch_bytes",
    "atf_prefill_chunk_cached", "atf_decode_workspace_bytes", "atf_decode",
    "atf_decode_kcache_bytes", "atf_decode_pack_k", "atf_decode_kcache",
    "atf_paged_page_bytes", "atf_decode_paged_workspace_bytes", "atf_paged_write", "atf_decode_paged",
    "atf_decode_paged_noalloc", "atf_decode_append_kv",
)
NOALLOC_SCRATCH_BYTES = 32 << 20  # ATF_NOALLOC_SCRATCH_BYTES


class AtfError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, _lib().atf_status_string(status).decode()))


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("librfw_atf.so is not built (expected at %s); run "
                           "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
    u64p = ctypes.POINTER(ctypes.c_uint64)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.atf_status_string.argtypes = [ctypes.c_int]
    lib.atf_status_string.restype = ctypes.c_char_p
    lib.atf_version.argtypes = []
    lib.atf_version.restype = ctypes.c_char_p
    lib.atf_window_table.argtypes = [i32, f64, f64, i64p]
    lib.atf_window_table.restype = ctypes.c_int
    lib.atf_skipped_pair_products.argtypes = [i64, i32, f64, f64, i32, i32, u64p]
    lib.atf_skipped_pair_products.restype = ctypes.c_int
    lib.atf_prefill_workspace_bytes.argtypes = [i32, i32, i64, i32, ctypes.c_int]
    lib.atf_prefill_workspace_bytes.restype = sz
    lib.atf_prefill_chunk_workspace_bytes.argtypes = [i32, i32, i32, i64, i64, i32, ctypes.c_int]
    lib.atf_prefill_chunk_workspace_bytes.restype = sz
    lib.atf_prefill.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, f64, f64, i32, i64,
                                ctypes.c_int, vp, sz, u64p, vp]
    lib.atf_prefill.restype = ctypes.c_int
    lib.atf_prefill_prepare_kv.argtypes = [vp, vp, i32, i32, i64, i32, i32, f64, i64, ctypes.c_int,
                                           vp, sz, vp]
    lib.atf_prefill_prepare_kv.restype = ctypes.c_int
    lib.atf_prefill_attend.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, f64, f64, i32, i64,
                                       ctypes.c_int, vp, sz, u64p, vp]
    lib.atf_prefill_attend.restype = ctypes.c_int
    lib.atf_prefill_chunk.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, i64, i32, i32, f64, f64, i32, i64,
                                      ctypes.c_int, vp, sz, u64p, vp]
    lib.atf_prefill_chunk.restype = ctypes.c_int
    lib.atf_prefill_cache_bytes.argtypes = [i32, i32, i64, i32]
    lib.atf_prefill_cache_bytes.restype = sz
    lib.atf_prefill_cache_append.argtypes = [vp, vp, i32, i32, i64, i64, i64, i32, i32, f64, i64, vp, sz, vp]
    lib.atf_prefill_cache_append.restype = ctypes.c_int
    lib.atf_prefill_cached_scratch_bytes.argtypes = [i32, i32, i32, i64, i64, i32]
    lib.atf_prefill_cached_scratch_bytes.restype = sz
    lib.atf_prefill_chunk_cached.argtypes = [vp, vp, i32, i32, i32, i64, i64, i64, i32, i32, f64, f64, i32, i64,
                                             vp, sz, vp, sz, u64p, vp]
    lib.atf_prefill_chunk_cached.restype = ctypes.c_int
    lib.atf_decode_workspace_bytes.argtypes = [i32, i32, i32, i64, i32]
    lib.atf_decode_workspace_bytes.restype = sz
    lib.atf_decode.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, f64, f64, i32, i64,
                               ctypes.c_int, vp, sz, u64p, vp]
    lib.atf_decode.restype = ctypes.c_int
    lib.atf_decode_kcache_bytes.argtypes = [i32, i32, i64, i32]
    lib.atf_decode_kcache_bytes.restype = sz
    lib.atf_decode_pack_k.argtypes = [vp, vp, i32, i32, i64, i64, i64, i32, i32, f64, i64, ctypes.c_int, vp]
    lib.atf_decode_pack_k.restype = ctypes.c_int
    lib.atf_decode_append_kv.argtypes = [vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, i32, f64, i64, ctypes.c_int,
                                         vp]
    lib.atf_decode_append_kv.restype = ctypes.c_int
    lib.atf_decode_kcache.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, i64, i32, i32, f64, f64, i32, i64,
                                      ctypes.c_int, vp, sz, u64p, vp]
    lib.atf_decode_kcache.restype = ctypes.c_int
    lib.atf_decode_paged_workspace_bytes.argtypes = [i32, i32, i32, i64, i32]
    lib.atf_decode_paged_workspace_bytes.restype = sz
    lib.atf_paged_page_bytes.argtypes = [i32, i32]
    lib.atf_paged_page_bytes.restype = sz
    lib.atf_paged_write.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i64, i32, i32, f64, i64, ctypes.c_int,
                                    vp]
    lib.atf_paged_write.restype = ctypes.c_int
    lib.atf_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, i32, i32, f64, f64, i32,
                                     i64,
                                     ctypes.c_int, vp, sz, u64p, vp]
    lib.atf_decode_paged.restype = ctypes.c_int
    lib.atf_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, i32, i32, f64,
                                             f64, i32, i64, ctypes.c_int, u64p, vp]
    lib.atf_decode_paged_noalloc.restype = ctypes.c_int
    _LIB = lib
    return lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


def _check(status: int, where: str):
    if status != ATF_OK:
        raise AtfError(status, where)


# ------------------------------------------------------------- host-only calls

def atf_version() -> str:
    return _lib().atf_version().decode()


def atf_window_table(d: int, rope_base: float, alpha: float) -> np.ndarray:
    W = np.zeros(max(d // 2, 1), dtype=np.int64)
    _check(_lib().atf_window_table(d, rope_base, alpha, W.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
           "atf_window_table")
    return W[: d // 2]


def atf_skipped_pair_products(S: int, d: int, rope_base: float, alpha: float, causal: int = 1,
                              is_decode: int = 0) -> int:
    out = ctypes.c_uint64(0)
    _check(_lib().atf_skipped_pair_products(S, d, rope_base, alpha, causal, is_decode, ctypes.byref(out)),
           "atf_skipped_pair_products")
    return int(out.value)


def atf_prefill_workspace_bytes(B: int, Hkv: int, S: int, d: int, dtype: int) -> int:
    return int(_lib().atf_prefill_workspace_bytes(B, Hkv, S, d, dtype))


def atf_prefill_chunk_workspace_bytes(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int, dtype: int) -> int:
    return int(_lib().atf_prefill_chunk_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, dtype))


def atf_prefill_cache_bytes(B: int, Hkv: int, S_cap: int, d: int) -> int:
    return int(_lib().atf_prefill_cache_bytes(B, Hkv, S_cap, d))


def atf_prefill_cached_scratch_bytes(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int) -> int:
    return int(_lib().atf_prefill_cached_scratch_bytes(B, Hq, Hkv, Sq, Sk, d))


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def atf_prefill_cache_append(k, v, cache, *, k_begin: int, cap: int, rope_base: float, pos0: int = 0,
                             rope_layout="neox"):
    """Write k, v [B,Hkv,n,d] (pre-RoPE, bf16) as keys k_begin .. k_begin+n-1
    of a prefill cache of capacity `cap` (a uint8 buffer of
    atf_prefill_cache_bytes bytes)."""
    B, Hkv, n, d = k.shape
    _check(_lib().atf_prefill_cache_append(_dev(k, "k"), _dev(v, "v"), B, Hkv, n, int(k_begin), int(cap), d,
                                           _layout_code(rope_layout), float(rope_base), int(pos0),
                                           _dev(cache, "cache"), _nbytes(cache), _stream(k.device)),
           "atf_prefill_cache_append")


def atf_prefill_chunk_cached(q, cache, out=None, *, Hkv: int, Sk: int, cap: int, rope_base: float, alpha: float,
                             causal: int = 1, pos0: int = 0, scratch=None, return_skipped: bool = False,
                             rope_layout="neox"):
    """Chunked prefill over the first Sk keys of a prefill cache: q [B,Hq,Sq,d]
    are the last Sq of those Sk tokens (query i at pos0+Sk-Sq+i)."""
    B, Hq, Sq, d = q.shape
    if out is None:
        out = _torch().empty_like(q)
    if scratch is None:
        scratch = workspace(atf_prefill_cached_scratch_bytes(B, Hq, Hkv, Sq, Sk, d), q.device, "prefill_scratch")
    skipped = ctypes.c_uint64(0)
    _check(_lib().atf_prefill_chunk_cached(_dev(q, "q"), _dev(out, "out"), B, Hq, Hkv, Sq, int(Sk), int(cap), d,
                                           _layout_code(rope_layout), float(rope_base), float(alpha), int(causal),
                                           int(pos0), _dev(cache, "cache"), _nbytes(cache),
                                           _dev(scratch, "scratch"), _nbytes(scratch),
                                           ctypes.byref(skipped) if return_skipped else None, _stream(q.device)),
           "atf_prefill_chunk_cached")
    return (out, int(skipped.value)) if return_skipped else out


def atf_decode_workspace_bytes(B: int, Hq: int, Hkv: int, S: int, d: int) -> int:
    return int(_lib().atf_decode_workspace_bytes(B, Hq, Hkv, S, d))


# ---------------------------------------------------------------- device calls

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATF_BF16
    if t.dtype == torch.float32:
        return ATF_F32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % t.dtype)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_WS = {}
_WS_RETIRED = []


def workspace(nbytes: int, device, tag: str):
    """A cached caller-owned workspace of at least nbytes on `device`, one per
    (device, stream, tag): calls queued on different streams never share
    scratch.  A buffer outgrown by a later call is kept alive (never freed),
    so work already queued on it still owns its memory.  Under HIP graph
    capture the cache is not used: the caller must pass its own buffer, whose
    lifetime it controls for as long as the graph may replay."""
    torch = _torch()
    if torch.device(device).type != "cuda":
        raise ValueError("tensors must be GPU tensors")
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError("no default workspace under graph capture: pass ws= / scratch= explicitly")
    key = (str(device), torch.cuda.current_stream(device).cuda_stream, tag)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _WS_RETIRED.append(ws)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


ROPE_LAYOUTS = {"neox": 0, "gptj": 1}


def _layout_code(rope_layout) -> int:
    """"neox" (pair p = dims p, p + d/2) -> 0, "gptj" (dims 2p, 2p + 1) -> 1;
    an int is passed through unchanged (the library checks it)."""
    if isinstance(rope_layout, str):
        if rope_layout not in ROPE_LAYOUTS:
            raise ValueError("rope_layout must be one of %s" % sorted(ROPE_LAYOUTS))
        return ROPE_LAYOUTS[rope_layout]
    return int(rope_layout)


def atf_prefill(q, k, v, out=None, *, rope_base: float, alpha: float, causal: int = 1, pos0: int = 0,
                ws=None, return_skipped: bool = False, rope_layout="neox"):
    """Causal windowed-RoPE prefill.  q [B,Hq,S,d], k/v [B,Hkv,S,d] (pre-RoPE)."""
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    code = _dtype_code(q)
    if out is None:
        out = _torch().empty_like(q)
    nbytes = atf_prefill_workspace_bytes(B, Hkv, S, d, code)
    if ws is None:
        ws = workspace(nbytes, q.device, "prefill")
    skipped = ctypes.c_uint64(0)
    _check(_lib().atf_prefill(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                              B, Hq, Hkv, S, d, _layout_code(rope_layout), float(rope_base), float(alpha), int(causal), int(pos0),
                              code, _dev(ws, "workspace"), ws.numel(),
                              ctypes.byref(skipped) if return_skipped else None, _stream(q.device)),
           "atf_prefill")
    return (out, int(skipped.value)) if return_skipped else out


def atf_prefill_prepare_kv(k, v, *, rope_base: float, pos0: int = 0, ws, rope_layout="neox"):
    B, Hkv, S, d = k.shape
    code = _dtype_code(k)
    _check(_lib().atf_prefill_prepare_kv(_dev(k, "k"), _dev(v, "v"), B, Hkv, S, d, _layout_code(rope_layout),
                                         float(rope_base),
                                         int(pos0), code, _dev(ws, "workspace"), ws.numel(),
                                         _stream(k.device)),
           "atf_prefill_prepare_kv")


def atf_prefill_attend(q, k, v, out, *, rope_base: float, alpha: float, causal: int = 1, pos0: int = 0,
                       ws, return_skipped: bool = False, rope_layout="neox"):
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    code = _dtype_code(q)
    skipped = ctypes.c_uint64(0)
    _check(_lib().atf_prefill_attend(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                                     B, Hq, Hkv, S, d, _layout_code(rope_layout), float(rope_base), float(alpha),
                                     int(causal), int(pos0), code, _dev(ws, "workspace"), ws.numel(),
                                     ctypes.byref(skipped) if return_skipped else None,
                                     _stream(q.device)),
           "atf_prefill_attend")
    return int(skipped.value) if return_skipped else None


def atf_prefill_chunk(q, k, v, out=None, *, rope_base: float, alpha: float, causal: int = 1, pos0: int = 0,
                      ws=None, return_skipped: bool = False, rope_layout="neox"):
    """Chunked prefill: q [B,Hq,Sq,d] are the last Sq of the Sk tokens whose
    keys/values k, v [B,Hkv,Sk,d] hold (pre-RoPE); query i sits at pos0+Sk-Sq+i."""
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    code = _dtype_code(q)
    if out is None:
        out = _torch().empty_like(q)
    nbytes = atf_prefill_chunk_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, code)
    if ws is None:
        ws = workspace(nbytes, q.device, "prefill")
    skipped = ctypes.c_uint64(0)
    _check(_lib().atf_prefill_chunk(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                                    B, Hq, Hkv, Sq, Sk, d, _layout_code(rope_layout), float(rope_base),
                                    float(alpha), int(causal), int(pos0), code, _dev(ws, "workspace"), ws.numel(),
                                    ctypes.byref(skipped) if return_skipped else None, _stream(q.device)),
           "atf_prefill_chunk")
    return (out, int(skipped.value)) if return_skipped else out


def atf_decode(q, k, v, out=None, *, rope_base: float, alpha: float, causal: int = 1, pos0: int = 0,
               ws=None, return_skipped: bool = False, rope_layout="neox"):
    """Windowed-RoPE decode: q [B,Hq,1,d] at position pos0+S over the cache k/v [B,Hkv,S,d]."""
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query per sequence")
    Hkv, S = k.shape[1], k.shape[2]
    code = _dtype_code(q)
    if out is None:
        out = _torch().empty_like(q)
    nbytes = atf_decode_workspace_bytes(B, Hq, Hkv, S, d)
    if ws is None:
        ws = workspace(nbytes, q.device, "decode")
    skipped = ctypes.c_uint64(0)
    _check(_lib().atf_decode(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                             B, Hq, Hkv, S, d, _layout_code(rope_layout), float(rope_base), float(alpha), int(causal), int(pos0),
                             code, _dev(ws, "workspace"), ws.numel(),
                             ctypes.byref(skipped) if return_skipped else None, _stream(q.device)),
           "atf_decode")
    return (out, int(skipped.value)) if return_skipped else out


def atf_decode_kcache_bytes(B: int, Hkv: int, cap: int, d: int) -> int:
    return int(_lib().atf_decode_kcache_bytes(B, Hkv, cap, d))


def atf_decode_pack_k(k, kcache, *, k_begin: int, cap: int, rope_base: float, pos0: int = 0, rope_layout="neox"):
    """Write k [B,Hkv,n,d] (pre-RoPE, bf16) as cache keys k_begin.. of kcache."""
    B, Hkv, n, d = k.shape
    _check(_lib().atf_decode_pack_k(_dev(k, "k"), _dev(kcache, "kcache"), B, Hkv, n, int(k_begin), int(cap), d,
                                    _layout_code(rope_layout), float(rope_base), int(pos0), _dtype_code(k), _stream(k.device)),
           "atf_decode_pack_k")


def atf_decode_append_kv(k, v, kcache, vcache, *, k_begin: int, cap: int, rope_base: float, pos0: int = 0,
                         rope_layout="neox"):
    """Write k, v [B,Hkv,n,d] (pre-RoPE, bf16) as entries k_begin.. of the key
    cache kcache and the value cache vcache [B,Hkv,cap,d] in one launch."""
    B, Hkv, n, d = k.shape
    _check(_lib().atf_decode_append_kv(_dev(k, "k"), _dev(v, "v"), _dev(kcache, "kcache"), _dev(vcache, "vcache"),
                                       B, Hkv, n, int(k_begin), int(cap), d, _layout_code(rope_layout),
                                       float(rope_base), int(pos0), _dtype_code(k), _stream(k.device)),
           "atf_decode_append_kv")


def atf_decode_kcache(q, kcache, v, out=None, *, S: int, rope_base: float, alpha: float, causal: int = 1,
                      pos0: int = 0, ws=None, return_skipped: bool = False, rope_layout="neox"):
    """Decode over the windowed key cache: q [B,Hq,1,d] at pos0+S, v [B,Hkv,cap,d]."""
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query per sequence")
    Hkv, cap = v.shape[1], v.shape[2]
    code = _dtype_code(q)
    if out is None:
        out = _torch().empty_like(q)
    nbytes = atf_decode_workspace_bytes(B, Hq, Hkv, S, d)
    if ws is None:
        ws = workspace(nbytes, q.device, "decode")
    skipped = ctypes.c_uint64(0)
    _check(_lib().atf_decode_kcache(_dev(q, "q"), _dev(kcache, "kcache"), _dev(v, "v"), _dev(out, "out"),
                                    B, Hq, Hkv, int(S), cap, d, _layout_code(rope_layout), float(rope_base),
                                    float(alpha), int(causal),
                                    int(pos0), code, _dev(ws, "workspace"), ws.numel(),
                                    ctypes.byref(skipped) if return_skipped else None, _stream(q.device)),
           "atf_decode_kcache")
    return (out, int(skipped.value)) if return_skipped else out


def atf_paged_page_bytes(Hkv: int, d: int) -> int:
    return int(_lib().atf_paged_page_bytes(Hkv, d))


def atf_decode_paged_workspace_bytes(B: int, Hq: int, Hkv: int, max_len: int, d: int) -> int:
    return int(_lib().atf_decode_paged_workspace_bytes(B, Hq, Hkv, max_len, d))


def _dev_i32(t, name):
    torch = _torch()
    if t.dtype != torch.int32:
        raise TypeError("%s must be int32" % name)
    return _dev(t, name)


def atf_paged_write(k, v, kpool, vpool, page_table, *, k_begin: int, rope_base: float, pos0: int = 0,
                    rope_layout="neox"):
    """Write tokens k_begin.. of every sequence (k, v [B,Hkv,n,d]) into their pages.
    page_table: int32 [B, max_pages] on the device; pools: one page = atf_paged_page_bytes."""
    B, Hkv, n, d = k.shape
    max_pages = page_table.shape[1]
    num_pages = kpool.numel() * kpool.element_size() // atf_paged_page_bytes(Hkv, d)
    _check(_lib().atf_paged_write(_dev(k, "k"), _dev(v, "v"), _dev(kpool, "kpool"), _dev(vpool, "vpool"),
                                  _dev_i32(page_table, "page_table"), max_pages, num_pages, B, Hkv, n, int(k_begin),
                                  d, _layout_code(rope_layout), float(rope_base), int(pos0), _dtype_code(k),
                                  _stream(k.device)),
           "atf_paged_write")


def atf_decode_paged(q, kpool, vpool, page_table, seq_lens, out=None, *, max_len: int, rope_base: float,
                     alpha: float, causal: int = 1, pos0: int = 0, ws=None, return_skipped: bool = False,
                     rope_layout="neox"):
    """Ragged decode over the paged cache: q [B,Hq,1,d]; seq_lens int32 [B] on the device."""
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query per sequence")
    max_pages = page_table.shape[1]
    Hkv = kpool.shape[1] if kpool.dim() >= 2 else None
    if Hkv is None:
        raise ValueError("kpool must be shaped [num_pages, Hkv, ...]")
    num_pages = kpool.shape[0]
    code = _dtype_code(q)
    if out is None:
        out = _torch().empty_like(q)
    nbytes = atf_decode_paged_workspace_bytes(B, Hq, Hkv, max_len, d)
    if ws is None:
        ws = workspace(nbytes, q.device, "decode")
    skipped = ctypes.c_uint64(0)
    _check(_lib().atf_decode_paged(_dev(q, "q"), _dev(kpool, "kpool"), _dev(vpool, "vpool"), _dev(out, "out"),
                                   _dev_i32(page_table, "page_table"), _dev_i32(seq_lens, "seq_lens"), max_pages,
                                   num_pages, B, Hq, Hkv, int(max_len), d, _layout_code(rope_layout),
                                   float(rope_base), float(alpha),
                                   int(causal), int(pos0), code, _dev(ws, "workspace"), ws.numel(),
                                   ctypes.byref(skipped) if return_skipped else None, _stream(q.device)),
           "atf_decode_paged")
    return (out, int(skipped.value)) if return_skipped else out


def atf_decode_paged_noalloc(q, kpool, vpool, page_table, seq_lens, out=None, *, max_len: int, rope_base: float,
                             alpha: float, causal: int = 1, pos0: int = 0, return_skipped: bool = False,
                             rope_layout="neox"):
    """atf_decode_paged with the library's own scratch (no workspace): for
    callers that cannot allocate.  Calls that overlap on one GPU race."""
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query per sequence")
    max_pages = page_table.shape[1]
    if kpool.dim() < 2:
        raise ValueError("kpool must be shaped [num_pages, Hkv, ...]")
    Hkv, num_pages = kpool.shape[1], kpool.shape[0]
    if out is None:
        out = _torch().empty_like(q)
    skipped = ctypes.c_uint64(0)
    _check(_lib().atf_decode_paged_noalloc(_dev(q, "q"), _dev(kpool, "kpool"), _dev(vpool, "vpool"),
                                           _dev(out, "out"), _dev_i32(page_table, "page_table"),
                                           _dev_i32(seq_lens, "seq_lens"), max_pages, num_pages, B, Hq, Hkv,
                                           int(max_len), d, _layout_code(rope_layout), float(rope_base),
                                           float(alpha), int(causal), int(pos0), _dtype_code(q),
                                           ctypes.byref(skipped) if return_skipped else None, _stream(q.device)),
           "atf_decode_paged_noalloc")
    return (out, int(skipped.value)) if return_skipped else out


ALPHA_INF = math.inf
