"""HIP graph capture of the hot-path entry points.

Called without a host-side count, every entry point is a chain of kernel
launches whose tables (windows, angles, split plan) travel by value in the
kernel arguments, and whose counter is cleared by a kernel, not a memset. So
a call records into a graph. Each test captures one call, then replays it
several times. Between replays it rewrites the inputs in place eagerly and
synchronises. Every replay must equal a fresh eager call on the same inputs,
bit for bit (the kernels are deterministic apart from the count).
"""
import pytest

from parity import log, require_gpu

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def env():
    require_gpu()
    import torch

    import rope_frequency_windowed_amd as atf
    from rope_frequency_windowed_amd import inputs
    return torch, atf, inputs


def capture(torch, fn):
    """Warm fn up on a side stream, then record it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def refill(torch, tensors, seed):
    gen = torch.Generator(device=tensors[0].device)
    gen.manual_seed(seed)
    for t in tensors:
        t.copy_(torch.randn(t.shape, generator=gen, device=t.device, dtype=torch.float32).to(t.dtype))


@pytest.mark.parametrize("d", [128, 256])
def test_graph_prefill(env, d):
    torch, atf, inputs = env
    B, Hq, Hkv, S, base, alpha = 1, 4, 2, 3000, 1e6, 1.0
    log("case: graph prefill d=%d S=%d" % (d, S))
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=torch.bfloat16, device=dev)
    nb = atf.atf_prefill_workspace_bytes(B, Hkv, S, d, atf.ATF_BF16)
    ws_g = torch.empty(nb, dtype=torch.uint8, device=dev)
    ws_e = torch.empty(nb, dtype=torch.uint8, device=dev)
    out_g, out_e = torch.empty_like(q), torch.empty_like(q)

    def step(ws, out):
        atf.atf_prefill_prepare_kv(k, v, rope_base=base, ws=ws)
        atf.atf_prefill_attend(q, k, v, out, rope_base=base, alpha=alpha, ws=ws)

    g = capture(torch, lambda: step(ws_g, out_g))
    for r in range(REPLAYS):
        refill(torch, [q, k, v], 50 + r)
        g.replay()
        torch.cuda.synchronize()
        step(ws_e, out_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay %d differs from the eager call" % r


def test_graph_decode(env):
    torch, atf, inputs = env
    B, Hq, Hkv, S, d, base, alpha = 2, 8, 2, 5000, 128, 1e6, 1.0
    log("case: graph decode S=%d" % S)
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=torch.bfloat16, device=dev)
    nb = atf.atf_decode_workspace_bytes(B, Hq, Hkv, S, d)
    ws_g = torch.empty(nb, dtype=torch.uint8, device=dev)
    ws_e = torch.empty(nb, dtype=torch.uint8, device=dev)
    out_g, out_e = torch.empty_like(q), torch.empty_like(q)
    g = capture(torch, lambda: atf.atf_decode(q, k, v, out_g, rope_base=base, alpha=alpha, ws=ws_g))
    for r in range(REPLAYS):
        refill(torch, [q, k, v], 60 + r)
        g.replay()
        torch.cuda.synchronize()
        atf.atf_decode(q, k, v, out_e, rope_base=base, alpha=alpha, ws=ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay %d differs from the eager call" % r


def test_graph_decode_kcache(env):
    torch, atf, inputs = env
    B, Hq, Hkv, S, cap, d, base, alpha = 2, 7, 1, 4000, 4096, 128, 1e6, 1.0
    log("case: graph key-cache decode S=%d" % S)
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=torch.bfloat16, device=dev)
    vcache = torch.zeros(B, Hkv, cap, d, dtype=torch.bfloat16, device=dev)
    kcache = torch.empty(atf.atf_decode_kcache_bytes(B, Hkv, cap, d), dtype=torch.uint8, device=dev)
    nb = atf.atf_decode_workspace_bytes(B, Hq, Hkv, S, d)
    ws_g = torch.empty(nb, dtype=torch.uint8, device=dev)
    ws_e = torch.empty(nb, dtype=torch.uint8, device=dev)
    out_g, out_e = torch.empty_like(q), torch.empty_like(q)

    def fill():
        atf.atf_decode_pack_k(k, kcache, k_begin=0, cap=cap, rope_base=base)
        vcache[:, :, :S].copy_(v)

    fill()
    g = capture(torch, lambda: atf.atf_decode_kcache(q, kcache, vcache, out_g, S=S, rope_base=base, alpha=alpha,
                                                     ws=ws_g))
    for r in range(REPLAYS):
        refill(torch, [q, k, v], 70 + r)
        fill()
        g.replay()
        torch.cuda.synchronize()
        atf.atf_decode_kcache(q, kcache, vcache, out_e, S=S, rope_base=base, alpha=alpha, ws=ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay %d differs from the eager call" % r


def test_graph_decode_paged_lengths_change(env):
    """The paged call reads page table and lengths from device memory, so one
    graph serves a batch whose lengths change between replays."""
    torch, atf, inputs = env
    Hq, Hkv, d, base, alpha, page = 4, 2, 128, 1e6, 1.0, 64
    max_len = 3000
    lens_per_replay = [[3000, 1200, 64], [2500, 1, 700], [64, 2999, 3000]]
    B = len(lens_per_replay[0])
    log("case: graph paged decode, lengths change per replay")
    dev = torch.device("cuda:0")
    max_pages = (max_len + page - 1) // page
    num_pages = B * max_pages
    gen = torch.Generator(device="cpu")
    gen.manual_seed(77)
    page_table = torch.randperm(num_pages, generator=gen).to(torch.int32).reshape(B, max_pages).to(dev)
    pb = atf.atf_paged_page_bytes(Hkv, d)
    kpool = torch.zeros(num_pages, Hkv, pb // Hkv, dtype=torch.uint8, device=dev)
    vpool = torch.zeros(num_pages, Hkv, pb // Hkv, dtype=torch.uint8, device=dev)
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, max_len, d, dtype=torch.bfloat16, device=dev)
    atf.atf_paged_write(k, v, kpool, vpool, page_table, k_begin=0, rope_base=base)
    seq_lens = torch.tensor(lens_per_replay[0], dtype=torch.int32, device=dev)
    nb = atf.atf_decode_paged_workspace_bytes(B, Hq, Hkv, max_len, d)
    ws_g = torch.empty(nb, dtype=torch.uint8, device=dev)
    ws_e = torch.empty(nb, dtype=torch.uint8, device=dev)
    out_g, out_e = torch.empty_like(q), torch.empty_like(q)

    def call(out, ws):
        atf.atf_decode_paged(q, kpool, vpool, page_table, seq_lens, out, max_len=max_len, rope_base=base,
                             alpha=alpha, ws=ws)

    g = capture(torch, lambda: call(out_g, ws_g))
    for r, lens in enumerate(lens_per_replay):
        seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        refill(torch, [q], 80 + r)
        g.replay()
        torch.cuda.synchronize()
        call(out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay %d (lens %s) differs from the eager call" % (r, lens)
