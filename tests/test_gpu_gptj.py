"""GPU parity of the GPT-J interleaved rotary layout (pair p = dims 2p, 2p+1)
on every entry point that reads q or k rows, through the C ABI, against the
fp64 oracle; plus the identity that the interleaved result equals the
half-split result on the same pairs stored in moved dims, bit for bit."""
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


def moved(x):
    """Dims (2p, 2p+1) -> (p, p+P): the half-split row holding the same pairs."""
    import torch
    return torch.cat([x[..., 0::2], x[..., 1::2]], dim=-1).contiguous()


PREFILL = [
    # B, Hq, Hkv, S, d, base, alpha, causal
    (1, 2, 1, 300, 64, 1e4, 1.0, 1),
    (1, 7, 1, 1000, 128, 1e6, 1.0, 1),
    (2, 4, 2, 777, 128, 1e6, 0.5, 1),
    (1, 28, 4, 2048, 128, 1e6, 2.0, 1),
    (1, 4, 2, 600, 128, 1e6, 1.0, 0),
    (1, 2, 1, 1, 128, 1e6, 1.0, 1),
    (1, 3, 1, 500, 64, 100.0, 0.3, 1),
    (1, 2, 1, 400, 128, 1e6, math.inf, 1),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,d,base,alpha,causal", PREFILL)
def test_gptj_prefill_bf16(env, B, Hq, Hkv, S, d, base, alpha, causal):
    torch, oracle, atf, inputs = env
    log("case: gptj prefill %s" % ((B, Hq, Hkv, S, d, base, alpha, causal),))
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill(q, k, v, rope_base=base, alpha=alpha, causal=causal, return_skipped=True,
                                   rope_layout="gptj")
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, causal=bool(causal), layout="gptj")
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, causal=bool(causal), layout="gptj")
    check_bf16(out.float().cpu().numpy(), ref, dense, "gptj prefill")
    assert skipped == ref_skipped


def test_gptj_prefill_equals_neox_on_moved_dims(env):
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(1, 7, 1, 3000, 3000, 128, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    a, sa = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0, return_skipped=True, rope_layout="gptj")
    b, sb = atf.atf_prefill(moved(q), moved(k), v, rope_base=1e6, alpha=1.0, return_skipped=True)
    torch.cuda.synchronize()
    assert sa == sb
    assert torch.equal(a, b)


def test_gptj_prefill_high_frequency_heavy(env):
    """Fast pairs scaled x1.5 where the interleaved layout stores them
    (pairs p < d/4 = dims 0 .. d/2 - 1)."""
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(1, 4, 1, 900, 900, 128, dtype=torch.bfloat16, device=torch.device("cuda:0"),
                              high_freq_scale=1.5, layout="gptj")
    out = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=0.5, rope_layout="gptj")
    torch.cuda.synchronize()
    ref, _ = oracle.attention(q, k, v, base=1e6, alpha=0.5, layout="gptj")
    dense, _ = oracle.attention(q, k, v, base=1e6, alpha=math.inf, layout="gptj")
    assert np.abs(dense - ref).max() > 0.05
    check_bf16(out.float().cpu().numpy(), ref, dense, "gptj hf", structured=True)


@pytest.mark.parametrize("Sq,Sk", [(100, 1000), (1, 777), (257, 5000)])
def test_gptj_chunk(env, Sq, Sk):
    torch, oracle, atf, inputs = env
    log("case: gptj chunk Sq=%d Sk=%d" % (Sq, Sk))
    q, k, v = inputs.make_qkv(1, 7, 1, Sq, Sk, 128, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill_chunk(q, k, v, rope_base=1e6, alpha=1.0, return_skipped=True, rope_layout="gptj")
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, q_pos0=Sk - Sq, k_pos0=0, layout="gptj")
    check_bf16(out.float().cpu().numpy(), ref, None, "gptj chunk")
    assert skipped == ref_skipped


@pytest.mark.parametrize("B,Hq,Hkv,S,d,causal", [(1, 1, 1, 256, 64, 1), (2, 4, 2, 333, 128, 1),
                                                 (1, 2, 1, 200, 64, 0)])
def test_gptj_prefill_fp32(env, B, Hq, Hkv, S, d, causal):
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=torch.float32, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill(q, k, v, rope_base=1e4, alpha=1.0, causal=causal, return_skipped=True,
                                   rope_layout="gptj")
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e4, alpha=1.0, causal=bool(causal), layout="gptj")
    check_f32(out.cpu().numpy(), ref, "gptj fp32")
    assert skipped == ref_skipped


DECODE = [
    # B, Hq, Hkv, S, d, base, alpha
    (2, 8, 2, 1000, 128, 1e6, 1.0),
    (1, 7, 1, 65, 128, 1e6, 1.0),
    (3, 28, 4, 4097, 128, 1e6, 2.0),
    (1, 4, 4, 5000, 64, 1e4, 0.5),
    (1, 16, 1, 777, 128, 1e6, 1.0),
    (2, 4, 1, 20000, 128, 1e6, 1.0),
    (1, 3, 1, 3000, 64, 100.0, 0.3),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,d,base,alpha", DECODE)
def test_gptj_decode_bf16(env, B, Hq, Hkv, S, d, base, alpha):
    torch, oracle, atf, inputs = env
    log("case: gptj decode %s" % ((B, Hq, Hkv, S, d, base, alpha),))
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_decode(q, k, v, rope_base=base, alpha=alpha, return_skipped=True, rope_layout="gptj")
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, q_pos0=S, k_pos0=0, layout="gptj")
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, q_pos0=S, k_pos0=0, layout="gptj")
    check_bf16(out.float().cpu().numpy(), ref, dense, "gptj decode")
    assert skipped == ref_skipped


def test_gptj_decode_equals_neox_on_moved_dims(env):
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(2, 28, 4, 1, 9000, 128, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    a = atf.atf_decode(q, k, v, rope_base=1e6, alpha=1.0, rope_layout="gptj")
    b = atf.atf_decode(moved(q), moved(k), v, rope_base=1e6, alpha=1.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_gptj_decode_fp32(env):
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(2, 4, 2, 1, 700, 64, dtype=torch.float32, device=torch.device("cuda:0"))
    out = atf.atf_decode(q, k, v, rope_base=1e4, alpha=1.0, rope_layout="gptj")
    torch.cuda.synchronize()
    ref, _ = oracle.attention(q, k, v, base=1e4, alpha=1.0, q_pos0=700, k_pos0=0, layout="gptj")
    check_f32(out.cpu().numpy(), ref, "gptj decode fp32")


@pytest.mark.parametrize("B,Hq,Hkv,S,cap,d", [(2, 8, 2, 1000, 1024, 128), (1, 4, 4, 5000, 5056, 64)])
def test_gptj_kcache(env, B, Hq, Hkv, S, cap, d):
    torch, oracle, atf, inputs = env
    log("case: gptj kcache %s" % ((B, Hq, Hkv, S, cap, d),))
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=torch.bfloat16, device=dev)
    kc = torch.empty(atf.atf_decode_kcache_bytes(B, Hkv, cap, d), dtype=torch.uint8, device=dev)
    atf.atf_decode_pack_k(k, kc, k_begin=0, cap=cap, rope_base=1e6, rope_layout="gptj")
    vc = torch.zeros(B, Hkv, cap, d, dtype=torch.bfloat16, device=dev)
    vc[:, :, :S] = v
    out, skipped = atf.atf_decode_kcache(q, kc, vc, S=S, rope_base=1e6, alpha=1.0, return_skipped=True,
                                         rope_layout="gptj")
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, q_pos0=S, k_pos0=0, layout="gptj")
    check_bf16(out.float().cpu().numpy(), ref, None, "gptj kcache")
    assert skipped == ref_skipped


def test_gptj_paged(env):
    torch, oracle, atf, inputs = env
    log("case: gptj paged")
    dev = torch.device("cuda:0")
    lens = [3000, 64, 1234]
    B, Hq, Hkv, d = 3, 8, 2, 128
    max_len = max(lens)
    max_pages = (max_len + 63) // 64
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, max_len, d, dtype=torch.bfloat16, device=dev)
    num_pages = B * max_pages + 3
    perm = np.random.default_rng(5).permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    pt = torch.as_tensor(perm.astype(np.int32), device=dev)
    pb = atf.atf_paged_page_bytes(Hkv, d)
    kpool = torch.zeros(num_pages, Hkv, pb // Hkv, dtype=torch.uint8, device=dev)
    vpool = torch.zeros(num_pages, Hkv, pb // Hkv, dtype=torch.uint8, device=dev)
    atf.atf_paged_write(k, v, kpool, vpool, pt, k_begin=0, rope_base=1e6, rope_layout="gptj")
    sl = torch.as_tensor(np.array(lens, dtype=np.int32), device=dev)
    out = atf.atf_decode_paged(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=1e6, alpha=1.0,
                               rope_layout="gptj")
    torch.cuda.synchronize()
    for b, S in enumerate(lens):
        ref, _ = oracle.attention(q[b:b + 1], k[b:b + 1, :, :S], v[b:b + 1, :, :S], base=1e6, alpha=1.0,
                                  q_pos0=S, k_pos0=0, layout="gptj")
        check_bf16(out[b:b + 1].float().cpu().numpy(), ref, None, "gptj paged seq %d" % b)


def test_gptj_prefill_workload_sampled(env):
    """S=32768 at the benchmark heads, sampled rows."""
    torch, oracle, atf, inputs = env
    from rope_frequency_windowed_amd.inputs import sample_rows
    B, Hq, Hkv, S, d = 1, 28, 4, 32768, 128
    log("case: gptj prefill S=32768 sampled")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0, return_skipped=True, rope_layout="gptj")
    torch.cuda.synchronize()
    assert skipped == B * Hq * atf.atf_skipped_pair_products(S, d, 1e6, 1.0, 1, 0)
    rows = np.array([(0, h, int(i)) for h in range(0, Hq, 4) for i in sample_rows(S, 4, seed=h)], dtype=np.int64)
    sel = torch.as_tensor(rows, device=q.device)
    qrows = q[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    got = out[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    kk, vv = k.float().cpu().numpy(), v.float().cpu().numpy()
    ref, _ = oracle.attention(qrows, kk, vv, base=1e6, alpha=1.0, rows=rows, q_shape=(B, Hq, S, d), layout="gptj")
    check_bf16(got, ref, None, "gptj 32K")
