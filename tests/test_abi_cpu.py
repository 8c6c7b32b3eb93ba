"""Host-side checks of librfw_atf.so that need no GPU: the library loads and
exports every symbol include/atf.h declares, its fp64 window table and closed
form agree with the (independently written) oracle, and every argument error
is reported before anything is launched."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import rope_frequency_windowed_amd as atf
from rope_frequency_windowed_amd import _binding as bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "atf.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(atf.LIB_PATH):
        from rope_frequency_windowed_amd import build
        build.build()
    return atf.library()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[a-z_ ]+\*?\s*\b(atf_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_binding_names():
    assert header_functions() == sorted(bnd.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert atf.atf_version().startswith("rfw-atf")


@pytest.mark.parametrize("d,base", [(64, 1e4), (128, 1e6), (128, 1e4), (16, 10.0), (2, 50.0)])
@pytest.mark.parametrize("alpha", [0.1, 0.5, 1.0, 2.0, 3.7, math.inf])
def test_window_table_matches_oracle(lib, orc, d, base, alpha):
    np.testing.assert_array_equal(atf.atf_window_table(d, base, alpha), orc.window_table(d, base, alpha))


@pytest.mark.parametrize("S", [1, 2, 7, 8, 100, 4097, 32768, 131072, 1 << 20])
@pytest.mark.parametrize("d,base,alpha", [(64, 1e4, 1.0), (128, 1e6, 0.5), (128, 1e6, 1.0),
                                          (128, 1e6, 2.0), (128, 1e6, math.inf)])
def test_closed_form_matches_oracle(lib, orc, S, d, base, alpha):
    for dec in (0, 1):
        assert atf.atf_skipped_pair_products(S, d, base, alpha, 1, dec) == \
            orc.skipped_closed_form(S, d, base, alpha, decode=bool(dec))


@pytest.mark.parametrize("S", [1, 2, 9, 40, 100])
@pytest.mark.parametrize("d,base,alpha", [(16, 10.0, 1.0), (8, 3.0, 0.5), (16, 10.0, math.inf)])
def test_noncausal_closed_form_matches_oracle(lib, orc, S, d, base, alpha):
    """Non-causal prefill: the library's closed form equals the oracle's
    enumeration of (i, j, p) with |i - j| > W_p, and twice the causal count;
    decode is unchanged."""
    rng = np.random.default_rng(S)
    q = rng.standard_normal((1, 1, S, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, S, d)).astype(np.float32)
    _, cnt = orc.attention(q, k, k, base=base, alpha=alpha, causal=False)
    got = atf.atf_skipped_pair_products(S, d, base, alpha, 0, 0)
    assert got == cnt == 2 * atf.atf_skipped_pair_products(S, d, base, alpha, 1, 0)
    assert atf.atf_skipped_pair_products(S, d, base, alpha, 0, 1) == atf.atf_skipped_pair_products(S, d, base, alpha, 1, 1)


def test_known_counts(lib):
    assert atf.atf_skipped_pair_products(256, 64, 1e4, 1.0) == 270074


def _call_prefill(lib, **kw):
    args = dict(q=16, k=32, v=48, out=64, B=1, Hq=4, Hkv=2, S=128, d=128, layout=0, base=1e6, alpha=1.0,
                causal=1, pos0=0, dtype=atf.ATF_BF16, ws=4096, ws_bytes=1, skipped=None, stream=None)
    args.update(kw)
    return lib.atf_prefill(ctypes.c_void_p(args["q"]), ctypes.c_void_p(args["k"]), ctypes.c_void_p(args["v"]),
                           ctypes.c_void_p(args["out"]), args["B"], args["Hq"], args["Hkv"], args["S"],
                           args["d"], args["layout"], args["base"], args["alpha"], args["causal"], args["pos0"],
                           args["dtype"], ctypes.c_void_p(args["ws"]), args["ws_bytes"], args["skipped"],
                           args["stream"])


def _call_decode(lib, **kw):
    args = dict(q=16, k=32, v=48, out=64, B=1, Hq=4, Hkv=2, S=128, d=128, layout=0, base=1e6, alpha=1.0,
                causal=1, pos0=0, dtype=atf.ATF_BF16, ws=4096, ws_bytes=1, skipped=None, stream=None)
    args.update(kw)
    return lib.atf_decode(ctypes.c_void_p(args["q"]), ctypes.c_void_p(args["k"]), ctypes.c_void_p(args["v"]),
                          ctypes.c_void_p(args["out"]), args["B"], args["Hq"], args["Hkv"], args["S"],
                          args["d"], args["layout"], args["base"], args["alpha"], args["causal"], args["pos0"],
                          args["dtype"], ctypes.c_void_p(args["ws"]), args["ws_bytes"], args["skipped"],
                          args["stream"])


# Every case below fails validation, so nothing reaches the GPU runtime.
BAD = [
    (dict(q=None), bnd.ATF_ERR_INVALID_ARG),
    (dict(k=None), bnd.ATF_ERR_INVALID_ARG),
    (dict(out=8), bnd.ATF_ERR_INVALID_ARG),            # misaligned
    (dict(B=0), bnd.ATF_ERR_INVALID_ARG),
    (dict(Hq=0), bnd.ATF_ERR_INVALID_ARG),
    (dict(Hq=5, Hkv=2), bnd.ATF_ERR_INVALID_ARG),      # Hq % Hkv != 0
    (dict(S=0), bnd.ATF_ERR_INVALID_ARG),
    (dict(d=63), bnd.ATF_ERR_INVALID_ARG),
    (dict(d=96), bnd.ATF_ERR_UNSUPPORTED),
    (dict(d=256), bnd.ATF_ERR_WORKSPACE),              # valid: stops at the workspace
    (dict(d=512), bnd.ATF_ERR_UNSUPPORTED),
    (dict(base=1.0), bnd.ATF_ERR_INVALID_ARG),
    (dict(base=float("inf")), bnd.ATF_ERR_INVALID_ARG),
    (dict(alpha=0.0), bnd.ATF_ERR_INVALID_ARG),
    (dict(alpha=-2.0), bnd.ATF_ERR_INVALID_ARG),
    (dict(alpha=float("nan")), bnd.ATF_ERR_INVALID_ARG),
    (dict(causal=0), bnd.ATF_ERR_WORKSPACE),           # valid (non-causal): stops at the workspace
    (dict(causal=2), bnd.ATF_ERR_INVALID_ARG),
    (dict(dtype=7), bnd.ATF_ERR_INVALID_ARG),
    (dict(pos0=-1), bnd.ATF_ERR_INVALID_ARG),
    (dict(pos0=(1 << 31) - 100), bnd.ATF_ERR_INVALID_ARG),
    (dict(ws=None), bnd.ATF_ERR_WORKSPACE),
    (dict(ws_bytes=1), bnd.ATF_ERR_WORKSPACE),         # undersized (valid otherwise)
    (dict(Hq=128, Hkv=1), bnd.ATF_ERR_UNSUPPORTED),    # group > 64
    (dict(layout=2), bnd.ATF_ERR_INVALID_ARG),         # rotary layout: 0 (NeoX) or 1 (GPT-J)
    (dict(layout=-1), bnd.ATF_ERR_INVALID_ARG),
    (dict(layout=1), bnd.ATF_ERR_WORKSPACE),           # valid (GPT-J): stops at the workspace
]


@pytest.mark.parametrize("kw,expect", BAD)
def test_prefill_rejects(lib, kw, expect):
    assert _call_prefill(lib, **kw) == expect


@pytest.mark.parametrize("kw,expect", BAD)
def test_decode_rejects(lib, kw, expect):
    assert _call_decode(lib, **kw) == expect


def test_workspace_sizes(lib):
    assert atf.atf_prefill_workspace_bytes(1, 4, 131072, 128, atf.ATF_BF16) == 256 + 2 * 4 * 131072 * 128 * 2
    assert atf.atf_prefill_workspace_bytes(1, 4, 100, 128, atf.ATF_BF16) == 256 + 2 * 4 * 128 * 128 * 2
    assert atf.atf_prefill_workspace_bytes(1, 1, 256, 64, atf.ATF_F32) == 256
    assert atf.atf_prefill_workspace_bytes(1, 1, 256, 96, atf.ATF_BF16) == 0
    # header, rotated queries (B*Hq rows of d bf16, rounded up to 256 bytes), partials
    ws = atf.atf_decode_workspace_bytes(8, 28, 4, 262144, 128)
    assert ws == 256 + 8 * 28 * 128 * 2 + 8 * 28 * 16 * 130 * 4  # 512 workgroups over 32 (sequence, kv head) units
    assert atf.atf_decode_workspace_bytes(1, 1, 1, 10, 128) == 256 + 256 + 1 * 1 * 1 * 130 * 4
    assert atf.atf_decode_workspace_bytes(1, 3, 1, 10, 64) == 256 + 512 + 3 * 1 * 66 * 4
    assert atf.atf_decode_workspace_bytes(1, 3, 2, 10, 128) == 0


def _split_extra(B, Hq, Sq, d, ns):
    """Partials of ns splits, then (16x16x32 kernel: d = 256, or d = 128 with
    at most 16 queries) the rotated queries at a 256-byte boundary."""
    part = B * Hq * Sq * ns * (d + 2) * 4
    if d == 256 or (d == 128 and Sq <= 16):
        part = (part + 255) // 256 * 256 + B * Hq * Sq * (d // 2) * 4
    return part


def test_chunk_workspace_sizes(lib):
    pre = atf.atf_prefill_workspace_bytes(1, 4, 32768, 128, atf.ATF_BF16)
    # 16 queries, 4 heads: one query tile per head, 512 // 4 = 128 capped at 64 splits
    assert atf.atf_prefill_chunk_workspace_bytes(1, 4, 4, 16, 32768, 128, atf.ATF_BF16) == \
        pre + _split_extra(1, 4, 16, 128, 64)
    # at most Sk / 256 splits (two 128-key tiles each)
    assert atf.atf_prefill_chunk_workspace_bytes(1, 4, 4, 17, 1000, 128, atf.ATF_BF16) == \
        atf.atf_prefill_workspace_bytes(1, 4, 1000, 128, atf.ATF_BF16) + 4 * 17 * 3 * 130 * 4
    # a chunk that fills the GPU by itself, fp32, or a too-short key range: no partials
    assert atf.atf_prefill_chunk_workspace_bytes(1, 28, 4, 32768, 32768, 128, atf.ATF_BF16) == \
        atf.atf_prefill_workspace_bytes(1, 4, 32768, 128, atf.ATF_BF16)
    assert atf.atf_prefill_chunk_workspace_bytes(1, 4, 4, 16, 32768, 128, atf.ATF_F32) == 256
    assert atf.atf_prefill_chunk_workspace_bytes(1, 4, 4, 16, 200, 128, atf.ATF_BF16) == \
        atf.atf_prefill_workspace_bytes(1, 4, 200, 128, atf.ATF_BF16)
    # 7 heads per kv head, 16 queries: head-packed work items (one per kv head)
    # leave 4 workgroups with work, so 64 splits; unpacked it would be 28 (18 splits)
    assert atf.atf_prefill_chunk_workspace_bytes(1, 28, 4, 16, 131072, 128, atf.ATF_BF16) == \
        atf.atf_prefill_workspace_bytes(1, 4, 131072, 128, atf.ATF_BF16) + _split_extra(1, 28, 16, 128, 64)
    # 4096 queries after 126976 cached tokens: 448 query-tile workgroups fill
    # 1.75 rounds of 256; four splits make 7 full rounds
    assert atf.atf_prefill_chunk_workspace_bytes(1, 28, 4, 4096, 131072, 128, atf.ATF_BF16) == \
        atf.atf_prefill_workspace_bytes(1, 4, 131072, 128, atf.ATF_BF16) + 28 * 4096 * 4 * 130 * 4
    # the same queries over a prefix shorter than three chunks: no split
    assert atf.atf_prefill_chunk_workspace_bytes(1, 28, 4, 4096, 16000, 128, atf.ATF_BF16) == \
        atf.atf_prefill_workspace_bytes(1, 4, 16000, 128, atf.ATF_BF16)
    # at most 16 queries (d = 128): 64-key tiles of the 16x16x32 kernel, so
    # Sk = 1000 allows 7 splits of two tiles (128-key tiles would allow 3)
    assert atf.atf_prefill_chunk_workspace_bytes(1, 28, 4, 16, 1000, 128, atf.ATF_BF16) == \
        atf.atf_prefill_workspace_bytes(1, 4, 1000, 128, atf.ATF_BF16) + _split_extra(1, 28, 16, 128, 7)
    assert atf.atf_prefill_chunk_workspace_bytes(1, 28, 4, 17, 1000, 128, atf.ATF_BF16) == \
        atf.atf_prefill_workspace_bytes(1, 4, 1000, 128, atf.ATF_BF16) + 28 * 17 * 3 * 130 * 4
    # d = 256: 64-key tiles, 128-query tiles
    assert atf.atf_prefill_chunk_workspace_bytes(1, 2, 1, 100, 1500, 256, atf.ATF_BF16) == \
        atf.atf_prefill_workspace_bytes(1, 1, 1500, 256, atf.ATF_BF16) + _split_extra(1, 2, 100, 256, 11)
    # d = 64 short chunks run on the 32x32 kernel, which rotates its own
    # queries: partials only (a whole number of split rows, at most 64 splits)
    extra = atf.atf_prefill_chunk_workspace_bytes(1, 4, 2, 16, 3000, 64, atf.ATF_BF16) - \
        atf.atf_prefill_workspace_bytes(1, 2, 3000, 64, atf.ATF_BF16)
    row = 4 * 16 * 66 * 4
    assert extra > 0 and extra % row == 0 and 1 < extra // row <= 64
    for bad in ((1, 3, 2, 16, 100, 128), (1, 4, 4, 0, 100, 128), (1, 4, 4, 101, 100, 128),
                (1, 4, 4, 16, 100, 96)):
        assert atf.atf_prefill_chunk_workspace_bytes(*bad, atf.ATF_BF16) == 0


def test_status_strings(lib):
    for code in range(5):
        assert lib.atf_status_string(code).decode().startswith("ATF_")


def test_python_binding_needs_gpu_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        atf.atf_prefill(q, q, q, rope_base=1e4, alpha=1.0)


def _call_chunk(lib, **kw):
    args = dict(q=16, k=32, v=48, out=64, B=1, Hq=4, Hkv=2, Sq=64, Sk=128, d=128, layout=0, base=1e6, alpha=1.0,
                causal=1, pos0=0, dtype=atf.ATF_BF16, ws=4096, ws_bytes=1, skipped=None, stream=None)
    args.update(kw)
    return lib.atf_prefill_chunk(ctypes.c_void_p(args["q"]), ctypes.c_void_p(args["k"]),
                                 ctypes.c_void_p(args["v"]), ctypes.c_void_p(args["out"]), args["B"],
                                 args["Hq"], args["Hkv"], args["Sq"], args["Sk"], args["d"], args["layout"], args["base"],
                                 args["alpha"], args["causal"], args["pos0"], args["dtype"],
                                 ctypes.c_void_p(args["ws"]), args["ws_bytes"], args["skipped"], args["stream"])


@pytest.mark.parametrize("kw,expect", [(dict((("Sk" if k == "S" else k), v) for k, v in kw.items()), e)
                                       for kw, e in BAD])
def test_chunk_rejects(lib, kw, expect):
    assert _call_chunk(lib, **kw) == expect


@pytest.mark.parametrize("kw", [dict(Sq=0), dict(Sq=-1), dict(Sq=129, Sk=128), dict(Sq=2, Sk=1)])
def test_chunk_rejects_bad_lengths(lib, kw):
    assert _call_chunk(lib, **kw) == bnd.ATF_ERR_INVALID_ARG


def test_kcache_bytes(lib):
    assert atf.atf_decode_kcache_bytes(8, 4, 262144, 128) == 8 * 4 * 262144 * 128 * 2
    assert atf.atf_decode_kcache_bytes(1, 1, 64, 64) == 64 * 64 * 2
    assert atf.atf_decode_kcache_bytes(2, 1, 128, 256) == 2 * 128 * 256 * 2
    for bad in [(1, 1, 100, 128), (1, 1, 0, 128), (0, 1, 64, 128), (1, 1, 64, 96), (1, 1, 1 << 31, 128),
                (1, 1, 64, 512)]:
        assert atf.atf_decode_kcache_bytes(*bad) == 0


def _call_pack(lib, **kw):
    args = dict(k=32, kc=4096, B=1, Hkv=2, n=10, k_begin=0, cap=128, d=128, layout=0, base=1e6, pos0=0,
                dtype=atf.ATF_BF16, stream=None)
    args.update(kw)
    return lib.atf_decode_pack_k(ctypes.c_void_p(args["k"]), ctypes.c_void_p(args["kc"]), args["B"], args["Hkv"],
                                 args["n"], args["k_begin"], args["cap"], args["d"], args["layout"], args["base"],
                                 args["pos0"],
                                 args["dtype"], args["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(k=None), bnd.ATF_ERR_INVALID_ARG), (dict(kc=None), bnd.ATF_ERR_INVALID_ARG),
    (dict(kc=4100), bnd.ATF_ERR_INVALID_ARG), (dict(n=0), bnd.ATF_ERR_INVALID_ARG),
    (dict(k_begin=-1), bnd.ATF_ERR_INVALID_ARG), (dict(cap=100), bnd.ATF_ERR_INVALID_ARG),
    (dict(k_begin=120, n=10), bnd.ATF_ERR_INVALID_ARG), (dict(d=63), bnd.ATF_ERR_INVALID_ARG),
    (dict(d=96), bnd.ATF_ERR_UNSUPPORTED), (dict(base=1.0), bnd.ATF_ERR_INVALID_ARG),
    (dict(pos0=-1), bnd.ATF_ERR_INVALID_ARG), (dict(pos0=(1 << 31) - 100), bnd.ATF_ERR_INVALID_ARG),
    (dict(dtype=atf.ATF_F32), bnd.ATF_ERR_UNSUPPORTED), (dict(dtype=5), bnd.ATF_ERR_INVALID_ARG),
    (dict(layout=3), bnd.ATF_ERR_INVALID_ARG),
])
def test_pack_rejects(lib, kw, expect):
    assert _call_pack(lib, **kw) == expect


def _call_append_kv(lib, **kw):
    args = dict(k=16, v=4096, kc=32, vc=8192, B=1, Hkv=2, n=10, k_begin=0, cap=128, d=128, layout=0, base=1e6,
                pos0=0, dtype=atf.ATF_BF16, stream=None)
    args.update(kw)
    return lib.atf_decode_append_kv(*(ctypes.c_void_p(args[x]) for x in ("k", "v", "kc", "vc")), args["B"],
                                    args["Hkv"], args["n"], args["k_begin"], args["cap"], args["d"], args["layout"],
                                    args["base"], args["pos0"], args["dtype"], args["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(k=None), bnd.ATF_ERR_INVALID_ARG), (dict(kc=None), bnd.ATF_ERR_INVALID_ARG),
    (dict(v=None), bnd.ATF_ERR_INVALID_ARG), (dict(vc=None), bnd.ATF_ERR_INVALID_ARG),
    (dict(v=4100), bnd.ATF_ERR_INVALID_ARG), (dict(vc=8200), bnd.ATF_ERR_INVALID_ARG),
    (dict(n=0), bnd.ATF_ERR_INVALID_ARG), (dict(k_begin=120, n=10), bnd.ATF_ERR_INVALID_ARG),
    (dict(cap=100), bnd.ATF_ERR_INVALID_ARG), (dict(d=96), bnd.ATF_ERR_UNSUPPORTED),
    (dict(dtype=atf.ATF_F32), bnd.ATF_ERR_UNSUPPORTED), (dict(layout=3), bnd.ATF_ERR_INVALID_ARG),
    (dict(pos0=-1), bnd.ATF_ERR_INVALID_ARG), (dict(base=0.5), bnd.ATF_ERR_INVALID_ARG),
])
def test_append_kv_rejects(lib, kw, expect):
    assert _call_append_kv(lib, **kw) == expect


def _call_kcache(lib, **kw):
    args = dict(q=16, kc=32, v=48, out=64, B=1, Hq=4, Hkv=2, S=128, cap=128, d=128, layout=0, base=1e6, alpha=1.0,
                causal=1, pos0=0, dtype=atf.ATF_BF16, ws=4096, ws_bytes=1, skipped=None, stream=None)
    args.update(kw)
    return lib.atf_decode_kcache(ctypes.c_void_p(args["q"]), ctypes.c_void_p(args["kc"]),
                                 ctypes.c_void_p(args["v"]), ctypes.c_void_p(args["out"]), args["B"],
                                 args["Hq"], args["Hkv"], args["S"], args["cap"], args["d"], args["layout"], args["base"],
                                 args["alpha"], args["causal"], args["pos0"], args["dtype"],
                                 ctypes.c_void_p(args["ws"]), args["ws_bytes"], args["skipped"], args["stream"])


@pytest.mark.parametrize("kw,expect", [(dict(((k if k != "k" else "kc"), v) for k, v in kw.items()), e)
                                       for kw, e in BAD if "S" not in kw])
def test_kcache_decode_rejects(lib, kw, expect):
    assert _call_kcache(lib, **kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(cap=100), bnd.ATF_ERR_INVALID_ARG), (dict(S=129), bnd.ATF_ERR_INVALID_ARG),
    (dict(S=0), bnd.ATF_ERR_INVALID_ARG), (dict(dtype=atf.ATF_F32), bnd.ATF_ERR_UNSUPPORTED),
    (dict(pos0=(1 << 31) - 130), bnd.ATF_ERR_INVALID_ARG),
])
def test_kcache_decode_rejects_layout(lib, kw, expect):
    assert _call_kcache(lib, **kw) == expect


def test_paged_page_bytes(lib):
    assert atf.atf_paged_page_bytes(4, 128) == 4 * 64 * 128 * 2
    assert atf.atf_paged_page_bytes(1, 64) == 64 * 64 * 2
    assert atf.atf_paged_page_bytes(0, 128) == 0 and atf.atf_paged_page_bytes(2, 96) == 0
    assert atf.atf_paged_page_bytes(2, 256) == 2 * 64 * 256 * 2


def _call_pwrite(lib, **kw):
    args = dict(k=16, v=32, kp=48, vp=64, pt=128, max_pages=4, num_pages=8, B=2, Hkv=2, n=10, k_begin=0, d=128,
                layout=0, base=1e6, pos0=0, dtype=atf.ATF_BF16, stream=None)
    args.update(kw)
    return lib.atf_paged_write(*(ctypes.c_void_p(args[x]) for x in ("k", "v", "kp", "vp", "pt")),
                               args["max_pages"], args["num_pages"], args["B"], args["Hkv"], args["n"],
                               args["k_begin"], args["d"], args["layout"], args["base"], args["pos0"], args["dtype"],
                               args["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(k=None), bnd.ATF_ERR_INVALID_ARG), (dict(pt=None), bnd.ATF_ERR_INVALID_ARG),
    (dict(pt=130), bnd.ATF_ERR_INVALID_ARG), (dict(vp=72), bnd.ATF_ERR_INVALID_ARG),
    (dict(n=0), bnd.ATF_ERR_INVALID_ARG), (dict(k_begin=250, n=10), bnd.ATF_ERR_INVALID_ARG),
    (dict(max_pages=0), bnd.ATF_ERR_INVALID_ARG), (dict(num_pages=0), bnd.ATF_ERR_INVALID_ARG),
    (dict(d=96), bnd.ATF_ERR_UNSUPPORTED), (dict(dtype=atf.ATF_F32), bnd.ATF_ERR_UNSUPPORTED),
    (dict(base=0.5), bnd.ATF_ERR_INVALID_ARG), (dict(pos0=-3), bnd.ATF_ERR_INVALID_ARG),
    (dict(layout=9), bnd.ATF_ERR_INVALID_ARG),
])
def test_paged_write_rejects(lib, kw, expect):
    assert _call_pwrite(lib, **kw) == expect


def _call_pdecode(lib, **kw):
    args = dict(q=16, kp=32, vp=48, out=64, pt=128, sl=256, max_pages=4, num_pages=8, B=2, Hq=4, Hkv=2,
                max_len=200, d=128, layout=0, base=1e6, alpha=1.0, causal=1, pos0=0, dtype=atf.ATF_BF16, ws=4096,
                ws_bytes=1, skipped=None, stream=None)
    args.update(kw)
    return lib.atf_decode_paged(*(ctypes.c_void_p(args[x]) for x in ("q", "kp", "vp", "out", "pt", "sl")),
                                args["max_pages"], args["num_pages"], args["B"], args["Hq"], args["Hkv"],
                                args["max_len"], args["d"], args["layout"], args["base"], args["alpha"], args["causal"],
                                args["pos0"], args["dtype"], ctypes.c_void_p(args["ws"]), args["ws_bytes"],
                                args["skipped"], args["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), bnd.ATF_ERR_INVALID_ARG), (dict(sl=None), bnd.ATF_ERR_INVALID_ARG),
    (dict(sl=258), bnd.ATF_ERR_INVALID_ARG), (dict(max_len=257), bnd.ATF_ERR_INVALID_ARG),
    (dict(max_len=0), bnd.ATF_ERR_INVALID_ARG), (dict(num_pages=0), bnd.ATF_ERR_INVALID_ARG),
    (dict(Hq=5), bnd.ATF_ERR_INVALID_ARG), (dict(d=96), bnd.ATF_ERR_UNSUPPORTED),
    (dict(causal=0), bnd.ATF_ERR_WORKSPACE),           # valid (non-causal): stops at the workspace
    (dict(dtype=atf.ATF_F32), bnd.ATF_ERR_UNSUPPORTED),
    (dict(alpha=float("nan")), bnd.ATF_ERR_INVALID_ARG), (dict(ws_bytes=1), bnd.ATF_ERR_WORKSPACE),
    (dict(layout=2), bnd.ATF_ERR_INVALID_ARG), (dict(layout=1), bnd.ATF_ERR_WORKSPACE),
])
def test_paged_decode_rejects(lib, kw, expect):
    assert _call_pdecode(lib, **kw) == expect


def _call_pdecode_noalloc(lib, **kw):
    args = dict(q=16, kp=32, vp=48, out=64, pt=128, sl=256, max_pages=4, num_pages=8, B=2, Hq=4, Hkv=2,
                max_len=200, d=128, layout=0, base=1e6, alpha=1.0, causal=1, pos0=0, dtype=atf.ATF_BF16,
                skipped=None, stream=None)
    args.update(kw)
    return lib.atf_decode_paged_noalloc(*(ctypes.c_void_p(args[x]) for x in ("q", "kp", "vp", "out", "pt", "sl")),
                                        args["max_pages"], args["num_pages"], args["B"], args["Hq"], args["Hkv"],
                                        args["max_len"], args["d"], args["layout"], args["base"], args["alpha"],
                                        args["causal"], args["pos0"], args["dtype"], args["skipped"], args["stream"])


def _noalloc_max_batch(Hq, Hkv, max_len, d):
    b = 1
    while atf.atf_decode_paged_workspace_bytes(b + 1, Hq, Hkv, max_len, d) <= bnd.NOALLOC_SCRATCH_BYTES:
        b += 1
    return b


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), bnd.ATF_ERR_INVALID_ARG), (dict(sl=None), bnd.ATF_ERR_INVALID_ARG),
    (dict(sl=258), bnd.ATF_ERR_INVALID_ARG), (dict(max_len=257), bnd.ATF_ERR_INVALID_ARG),
    (dict(max_len=0), bnd.ATF_ERR_INVALID_ARG), (dict(num_pages=0), bnd.ATF_ERR_INVALID_ARG),
    (dict(Hq=5), bnd.ATF_ERR_INVALID_ARG), (dict(d=96), bnd.ATF_ERR_UNSUPPORTED),
    (dict(dtype=atf.ATF_F32), bnd.ATF_ERR_UNSUPPORTED), (dict(alpha=float("nan")), bnd.ATF_ERR_INVALID_ARG),
    (dict(layout=2), bnd.ATF_ERR_INVALID_ARG),
    # beyond the library's scratch: rejected on the host, before any HIP call
    (dict(B=18, Hq=28, Hkv=4, max_len=262144, max_pages=4096), bnd.ATF_ERR_WORKSPACE),
    (dict(B=16, Hq=64, Hkv=1, max_len=262144, max_pages=4096, d=256), bnd.ATF_ERR_WORKSPACE),
])
def test_paged_decode_noalloc_rejects(lib, kw, expect):
    assert _call_pdecode_noalloc(lib, **kw) == expect


def test_noalloc_scratch_limit():
    """The stated limit: at Hq=28, Hkv=4, d=128 the library's 32 MiB scratch
    holds a batch of 17 sequences and no more."""
    assert _noalloc_max_batch(28, 4, 262144, 128) == 17
    assert atf.atf_decode_paged_workspace_bytes(17, 28, 4, 262144, 128) <= 32 << 20
    assert atf.atf_decode_paged_workspace_bytes(18, 28, 4, 262144, 128) > 32 << 20


def test_probe_library_exports_and_checks_arguments():
    """The microbenchmark library exports what include/atf_probes.h declares
    and rejects bad arguments on the host (nothing is launched)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    hdr = open(os.path.join(root, "include", "atf_probes.h")).read()
    names = set(re.findall(r"^int (atf_probe_\w+)\(", hdr, re.M))
    assert names == {"atf_probe_mfma_bf16", "atf_probe_hbm_read"}
    from rope_frequency_windowed_amd import probes
    lib = probes.library()
    for n in names:
        assert hasattr(lib, n)
    assert lib.atf_probe_mfma_bf16(None, None, 1, 1, None) == 1
    assert lib.atf_probe_mfma_bf16(16, 32, 0, 1, None) == 1
    assert lib.atf_probe_hbm_read(16, 100, 32, 1, None) == 1      # size not a multiple of 256 KiB
    assert lib.atf_probe_hbm_read(8, 1 << 18, 32, 1, None) == 1   # misaligned


def test_prefill_cache_sizes(lib):
    assert atf.atf_prefill_cache_bytes(1, 4, 3000, 128) == 2 * 4 * 3072 * 128 * 2
    assert atf.atf_prefill_cache_bytes(2, 1, 128, 64) == 2 * 2 * 128 * 64 * 2
    assert atf.atf_prefill_cache_bytes(1, 4, 3000, 96) == 0
    assert atf.atf_prefill_cache_bytes(1, 4, 0, 128) == 0
    # scratch: counter, plus the partials (and rotated queries) of the same
    # split the chunk call plans
    assert atf.atf_prefill_cached_scratch_bytes(1, 28, 4, 16, 131072, 128) == 256 + _split_extra(1, 28, 16, 128, 64)
    assert _split_extra(1, 28, 16, 128, 64) == 28 * 16 * 64 * 130 * 4 + 28 * 16 * 64 * 4
    assert atf.atf_prefill_cached_scratch_bytes(1, 28, 4, 32768, 32768, 128) == 256
    assert atf.atf_prefill_cached_scratch_bytes(1, 28, 4, 17, 16, 128) == 0
    assert atf.atf_prefill_cached_scratch_bytes(1, 28, 3, 16, 100, 128) == 0
    for args in ((1, 28, 4, 16, 131072, 128), (1, 2, 1, 100, 1500, 256), (1, 4, 4, 17, 1000, 128)):
        B, Hq, Hkv, Sq, Sk, d = args
        assert atf.atf_prefill_cached_scratch_bytes(*args) - 256 == \
            atf.atf_prefill_chunk_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, atf.ATF_BF16) - \
            atf.atf_prefill_workspace_bytes(B, Hkv, Sk, d, atf.ATF_BF16)


def _call_append(lib, **kw):
    args = dict(k=16, v=32, B=1, Hkv=2, n=64, k_begin=0, cap=1000, d=128, layout=0, base=1e6, pos0=0,
                cache=4096, cache_bytes=1, stream=None)
    args.update(kw)
    return lib.atf_prefill_cache_append(ctypes.c_void_p(args["k"]), ctypes.c_void_p(args["v"]), args["B"],
                                        args["Hkv"], args["n"], args["k_begin"], args["cap"], args["d"],
                                        args["layout"], args["base"], args["pos0"], ctypes.c_void_p(args["cache"]),
                                        args["cache_bytes"], args["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(), bnd.ATF_ERR_WORKSPACE),                   # valid: stops at the cache size
    (dict(n=0), bnd.ATF_ERR_INVALID_ARG),
    (dict(k_begin=-1), bnd.ATF_ERR_INVALID_ARG),
    (dict(k_begin=937), bnd.ATF_ERR_INVALID_ARG),      # k_begin + n > cap
    (dict(k_begin=936), bnd.ATF_ERR_WORKSPACE),        # ends exactly at cap
    (dict(k=None), bnd.ATF_ERR_INVALID_ARG),
    (dict(v=8), bnd.ATF_ERR_INVALID_ARG),
    (dict(d=96), bnd.ATF_ERR_UNSUPPORTED),
    (dict(layout=3), bnd.ATF_ERR_INVALID_ARG),
    (dict(base=0.5), bnd.ATF_ERR_INVALID_ARG),
    (dict(cache=None), bnd.ATF_ERR_WORKSPACE),
    (dict(pos0=(1 << 31) - 500), bnd.ATF_ERR_INVALID_ARG),
])
def test_cache_append_rejects(lib, kw, expect):
    assert _call_append(lib, **kw) == expect


def _call_cached(lib, **kw):
    args = dict(q=16, out=32, B=1, Hq=4, Hkv=2, Sq=64, Sk=500, cap=1000, d=128, layout=0, base=1e6, alpha=1.0,
                causal=1, pos0=0, cache=4096, cache_bytes=2 * 2 * 1024 * 128 * 2, scratch=8192, scratch_bytes=1,
                skipped=None, stream=None)
    args.update(kw)
    return lib.atf_prefill_chunk_cached(ctypes.c_void_p(args["q"]), ctypes.c_void_p(args["out"]), args["B"],
                                        args["Hq"], args["Hkv"], args["Sq"], args["Sk"], args["cap"], args["d"],
                                        args["layout"], args["base"], args["alpha"], args["causal"], args["pos0"],
                                        ctypes.c_void_p(args["cache"]), args["cache_bytes"],
                                        ctypes.c_void_p(args["scratch"]), args["scratch_bytes"], args["skipped"],
                                        args["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(), bnd.ATF_ERR_WORKSPACE),                   # valid: stops at the scratch size
    (dict(Sq=0), bnd.ATF_ERR_INVALID_ARG),
    (dict(Sq=501), bnd.ATF_ERR_INVALID_ARG),           # Sq > Sk
    (dict(Sk=1001), bnd.ATF_ERR_INVALID_ARG),          # Sk > cap
    (dict(Hq=5), bnd.ATF_ERR_INVALID_ARG),
    (dict(q=None), bnd.ATF_ERR_INVALID_ARG),
    (dict(out=40), bnd.ATF_ERR_INVALID_ARG),
    (dict(alpha=float("nan")), bnd.ATF_ERR_INVALID_ARG),
    (dict(causal=3), bnd.ATF_ERR_INVALID_ARG),
    (dict(layout=5), bnd.ATF_ERR_INVALID_ARG),
    (dict(d=96), bnd.ATF_ERR_UNSUPPORTED),
    (dict(cache_bytes=2 * 2 * 1024 * 128 * 2 - 1), bnd.ATF_ERR_WORKSPACE),
    (dict(cache=None), bnd.ATF_ERR_WORKSPACE),
    (dict(scratch=None, scratch_bytes=256), bnd.ATF_ERR_WORKSPACE),
    (dict(scratch_bytes=255), bnd.ATF_ERR_WORKSPACE),
])
def test_chunk_cached_rejects(lib, kw, expect):
    assert _call_cached(lib, **kw) == expect
