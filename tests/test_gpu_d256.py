"""GPU parity at head dim d = 256 (128 rotary pairs, so a wave holds two
windows per lane and the prefill kernel runs 4-wave workgroups with 64-key
tiles) on every entry point, through the C ABI, against the fp64 oracle.
Base 1e4 puts W_64 at 629, so the sequences below cut pairs past lane 63."""
import math

import numpy as np
import pytest

from parity import check_bf16, check_f32, log, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    require_gpu()
    import torch

    import oracle
    import rope_frequency_windowed_amd as atf
    from rope_frequency_windowed_amd import inputs
    oracle.build()
    return torch, oracle, atf, inputs


def test_pairs_past_lane_63_are_cut(env):
    """The sizes below really exercise the second window half."""
    torch, oracle, atf, _ = env
    W = atf.atf_window_table(256, 1e4, 1.0)
    assert W[64] < 1000 and W[80] < 2500


PREFILL = [
    # B, Hq, Hkv, S, base, alpha, causal, layout
    (1, 2, 1, 2000, 1e4, 1.0, 1, "neox"),
    (1, 4, 2, 777, 1e4, 0.5, 1, "neox"),
    (2, 3, 1, 1500, 1e6, 1.0, 1, "neox"),
    (1, 2, 2, 129, 1e4, 1.0, 1, "neox"),
    (1, 1, 1, 1, 1e4, 1.0, 1, "neox"),
    (1, 2, 1, 1200, 1e4, 1.0, 0, "neox"),
    (1, 2, 1, 1800, 1e4, 2.0, 1, "gptj"),
    (1, 2, 1, 500, 1e4, math.inf, 1, "neox"),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,base,alpha,causal,layout", PREFILL)
def test_d256_prefill_bf16(env, B, Hq, Hkv, S, base, alpha, causal, layout):
    torch, oracle, atf, inputs = env
    log("case: d256 prefill %s" % ((B, Hq, Hkv, S, base, alpha, causal, layout),))
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, 256, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill(q, k, v, rope_base=base, alpha=alpha, causal=causal, return_skipped=True,
                                   rope_layout=layout)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, causal=bool(causal), layout=layout)
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, causal=bool(causal), layout=layout)
    check_bf16(out.float().cpu().numpy(), ref, dense, "d256 prefill")
    assert skipped == ref_skipped
    assert skipped == B * Hq * atf.atf_skipped_pair_products(S, 256, base, alpha, causal, 0)


def test_d256_prefill_high_frequency_heavy(env):
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(1, 2, 1, 1000, 1000, 256, dtype=torch.bfloat16, device=torch.device("cuda:0"),
                              high_freq_scale=1.5)
    out = atf.atf_prefill(q, k, v, rope_base=1e4, alpha=0.5)
    torch.cuda.synchronize()
    ref, _ = oracle.attention(q, k, v, base=1e4, alpha=0.5)
    dense, _ = oracle.attention(q, k, v, base=1e4, alpha=math.inf)
    assert np.abs(dense - ref).max() > 0.05
    check_bf16(out.float().cpu().numpy(), ref, dense, "d256 hf", structured=True)


@pytest.mark.parametrize("Sq,Sk", [(100, 1500), (1, 700)])
def test_d256_chunk(env, Sq, Sk):
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(1, 2, 1, Sq, Sk, 256, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill_chunk(q, k, v, rope_base=1e4, alpha=1.0, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e4, alpha=1.0, q_pos0=Sk - Sq, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, None, "d256 chunk")
    assert skipped == ref_skipped


@pytest.mark.parametrize("S,causal", [(300, 1), (200, 0)])
def test_d256_prefill_fp32(env, S, causal):
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(1, 2, 1, S, S, 256, dtype=torch.float32, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill(q, k, v, rope_base=1e4, alpha=0.5, causal=causal, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e4, alpha=0.5, causal=bool(causal))
    check_f32(out.cpu().numpy(), ref, "d256 fp32")
    assert skipped == ref_skipped


DECODE = [
    # B, Hq, Hkv, S, base, alpha, layout
    (2, 8, 2, 3000, 1e4, 1.0, "neox"),
    (1, 4, 1, 65, 1e4, 1.0, "neox"),
    (1, 16, 2, 20000, 1e6, 1.0, "neox"),
    (1, 4, 4, 5000, 1e4, 0.5, "gptj"),
    (2, 4, 1, 2049, 1e4, math.inf, "neox"),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,base,alpha,layout", DECODE)
def test_d256_decode_bf16(env, B, Hq, Hkv, S, base, alpha, layout):
    torch, oracle, atf, inputs = env
    log("case: d256 decode %s" % ((B, Hq, Hkv, S, base, alpha, layout),))
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, 256, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_decode(q, k, v, rope_base=base, alpha=alpha, return_skipped=True, rope_layout=layout)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, q_pos0=S, k_pos0=0, layout=layout)
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, q_pos0=S, k_pos0=0, layout=layout)
    check_bf16(out.float().cpu().numpy(), ref, dense, "d256 decode")
    assert skipped == ref_skipped


def test_d256_decode_fp32(env):
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(1, 4, 2, 1, 900, 256, dtype=torch.float32, device=torch.device("cuda:0"))
    out = atf.atf_decode(q, k, v, rope_base=1e4, alpha=1.0)
    torch.cuda.synchronize()
    ref, _ = oracle.attention(q, k, v, base=1e4, alpha=1.0, q_pos0=900, k_pos0=0)
    check_f32(out.cpu().numpy(), ref, "d256 decode fp32")


@pytest.mark.parametrize("S,cap,layout", [(3000, 3008, "neox"), (777, 1024, "gptj")])
def test_d256_kcache(env, S, cap, layout):
    torch, oracle, atf, inputs = env
    log("case: d256 kcache S=%d" % S)
    dev = torch.device("cuda:0")
    B, Hq, Hkv, d = 2, 8, 2, 256
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=torch.bfloat16, device=dev)
    kc = torch.empty(atf.atf_decode_kcache_bytes(B, Hkv, cap, d), dtype=torch.uint8, device=dev)
    atf.atf_decode_pack_k(k, kc, k_begin=0, cap=cap, rope_base=1e4, rope_layout=layout)
    vc = torch.zeros(B, Hkv, cap, d, dtype=torch.bfloat16, device=dev)
    vc[:, :, :S] = v
    out, skipped = atf.atf_decode_kcache(q, kc, vc, S=S, rope_base=1e4, alpha=1.0, return_skipped=True,
                                         rope_layout=layout)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e4, alpha=1.0, q_pos0=S, k_pos0=0, layout=layout)
    check_bf16(out.float().cpu().numpy(), ref, None, "d256 kcache")
    assert skipped == ref_skipped


def test_d256_paged(env):
    torch, oracle, atf, inputs = env
    log("case: d256 paged")
    dev = torch.device("cuda:0")
    lens = [2500, 64, 1001]
    B, Hq, Hkv, d = 3, 4, 2, 256
    max_len = max(lens)
    max_pages = (max_len + 63) // 64
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, max_len, d, dtype=torch.bfloat16, device=dev)
    num_pages = B * max_pages + 2
    perm = np.random.default_rng(9).permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    pt = torch.as_tensor(perm.astype(np.int32), device=dev)
    pb = atf.atf_paged_page_bytes(Hkv, d)
    kpool = torch.zeros(num_pages, Hkv, pb // Hkv, dtype=torch.uint8, device=dev)
    vpool = torch.zeros(num_pages, Hkv, pb // Hkv, dtype=torch.uint8, device=dev)
    atf.atf_paged_write(k, v, kpool, vpool, pt, k_begin=0, rope_base=1e4)
    sl = torch.as_tensor(np.array(lens, dtype=np.int32), device=dev)
    out, skipped = atf.atf_decode_paged(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=1e4, alpha=1.0,
                                        return_skipped=True)
    torch.cuda.synchronize()
    total = 0
    for b, S in enumerate(lens):
        ref, sk = oracle.attention(q[b:b + 1], k[b:b + 1, :, :S], v[b:b + 1, :, :S], base=1e4, alpha=1.0,
                                   q_pos0=S, k_pos0=0)
        check_bf16(out[b:b + 1].float().cpu().numpy(), ref, None, "d256 paged seq %d" % b)
        total += sk
    assert skipped == total


def test_d256_prefill_sampled_long(env):
    """S=16384, 8 query heads over 2 kv heads, base 1e6: sampled rows."""
    torch, oracle, atf, inputs = env
    from rope_frequency_windowed_amd.inputs import sample_rows
    B, Hq, Hkv, S, d = 1, 8, 2, 16384, 256
    log("case: d256 prefill S=16384 sampled")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0, return_skipped=True)
    torch.cuda.synchronize()
    assert skipped == B * Hq * atf.atf_skipped_pair_products(S, d, 1e6, 1.0, 1, 0)
    from rope_frequency_windowed_amd.inputs import tile_edge_rows
    # seeded rows plus the edges of 128-query tiles (this kernel's query tile)
    rows = np.array([(0, h, int(i)) for h in range(Hq)
                     for i in sorted(set(sample_rows(S, 3, seed=h)) | set(tile_edge_rows(S, 1, seed=h, tile=128)))],
                    dtype=np.int64)
    sel = torch.as_tensor(rows, device=q.device)
    qrows = q[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    got = out[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    kk, vv = k.float().cpu().numpy(), v.float().cpu().numpy()
    ref, _ = oracle.attention(qrows, kk, vv, base=1e6, alpha=1.0, rows=rows, q_shape=(B, Hq, S, d))
    dense, _ = oracle.attention(qrows, kk, vv, base=1e6, alpha=math.inf, rows=rows, q_shape=(B, Hq, S, d))
    check_bf16(got, ref, dense, "d256 16K")
