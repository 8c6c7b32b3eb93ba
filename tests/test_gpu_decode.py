"""GPU parity of the decode path (through the C ABI) against the fp64 oracle."""
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


def run_decode(env, B, Hq, Hkv, S, d, base, alpha, dtype, pos0=0, hf=None):
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=dtype, device=dev, high_freq_scale=hf)
    out, skipped = atf.atf_decode(q, k, v, rope_base=base, alpha=alpha, pos0=pos0, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, q_pos0=pos0 + S, k_pos0=pos0)
    return q, k, v, out, skipped, ref, ref_skipped


DECODE_BF16 = [
    # B, Hq, Hkv, S, d, base, alpha
    (2, 8, 2, 1000, 128, 1e6, 1.0),
    (1, 7, 1, 300, 128, 1e6, 1.0),
    (3, 28, 4, 4097, 128, 1e6, 2.0),
    (1, 2, 1, 1, 128, 1e6, 1.0),
    (1, 2, 1, 63, 128, 1e6, 1.0),
    (1, 2, 1, 65, 64, 1e4, 1.0),
    (1, 4, 4, 5000, 64, 1e4, 0.5),
    (1, 16, 1, 777, 128, 1e6, 1.0),     # two slabs of 8 query heads
    (1, 3, 1, 2000, 128, 1e6, math.inf),
    (2, 4, 1, 20000, 128, 1e6, 1.0),    # many splits
]


@pytest.mark.parametrize("B,Hq,Hkv,S,d,base,alpha", DECODE_BF16)
def test_decode_bf16(env, B, Hq, Hkv, S, d, base, alpha):
    torch, oracle, atf, _ = env
    log("case: decode bf16 %s" % ((B, Hq, Hkv, S, d, base, alpha),))
    q, k, v, out, skipped, ref, ref_skipped = run_decode(env, B, Hq, Hkv, S, d, base, alpha, torch.bfloat16)
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, q_pos0=S, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, dense, "decode %s" % ((B, Hq, Hkv, S, d),))
    assert skipped == ref_skipped
    assert skipped == B * Hq * atf.atf_skipped_pair_products(S, d, base, alpha, 1, 1)


@pytest.mark.parametrize("alpha", [0.5, 1.0])
def test_decode_high_frequency_heavy(env, alpha):
    torch, oracle, atf, _ = env
    log("case: decode hf alpha=%g" % alpha)
    q, k, v, out, skipped, ref, ref_skipped = run_decode(env, 1, 7, 1, 3000, 128, 1e6, alpha,
                                                         torch.bfloat16, hf=1.5)
    dense, _ = oracle.attention(q, k, v, base=1e6, alpha=math.inf, q_pos0=3000, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, dense, "decode hf", structured=True)
    assert skipped == ref_skipped


@pytest.mark.parametrize("pos0", [1 << 20, 1 << 24])
def test_decode_position_shift(env, pos0):
    torch, oracle, atf, _ = env
    log("case: decode pos0=%d" % pos0)
    q, k, v, out, skipped, ref, ref_skipped = run_decode(env, 2, 7, 1, 2500, 128, 1e6, 1.0,
                                                         torch.bfloat16, pos0=pos0)
    check_bf16(out.float().cpu().numpy(), ref, None, "decode pos0=%d" % pos0)
    assert skipped == ref_skipped


@pytest.mark.parametrize("B,Hq,Hkv,S,d", [(1, 4, 2, 300, 64), (2, 7, 1, 1000, 128)])
def test_decode_fp32(env, B, Hq, Hkv, S, d):
    torch, oracle, atf, _ = env
    log("case: decode fp32 %s" % ((B, Hq, Hkv, S, d),))
    q, k, v, out, skipped, ref, ref_skipped = run_decode(env, B, Hq, Hkv, S, d, 1e6, 1.0, torch.float32)
    check_f32(out.cpu().numpy(), ref, "decode fp32")
    assert skipped == ref_skipped


def test_decode_workload_full(env):
    """B=8 sequences, query at 262144 after a 262144-key cache, Hq=28, Hkv=4,
    d=128, base 1e6, alpha 1 -- every one of the 224 query rows vs the oracle."""
    torch, oracle, atf, _ = env
    log("case: decode workload S=262144 (all 224 rows)")
    q, k, v, out, skipped, ref, ref_skipped = run_decode(env, 8, 28, 4, 262144, 128, 1e6, 1.0, torch.bfloat16)
    dense, _ = oracle.attention(q, k, v, base=1e6, alpha=math.inf, q_pos0=262144, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, dense, "decode 256K")
    assert skipped == ref_skipped == 8 * 28 * atf.atf_skipped_pair_products(262144, 128, 1e6, 1.0, 1, 1)


@pytest.mark.parametrize("B,Hq,Hkv,S,d", [(2, 4, 4, 3000, 128),     # plain multi-head (group 1)
                                          (1, 64, 1, 2000, 64),     # the largest group: 8 slabs of 8 heads
                                          (16, 8, 2, 700, 128)])    # many sequences
def test_decode_group_and_batch_edges(env, B, Hq, Hkv, S, d):
    torch, oracle, atf, inputs = env
    log("case: decode edges %s" % ((B, Hq, Hkv, S, d),))
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_decode(q, k, v, rope_base=1e4, alpha=1.0, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e4, alpha=1.0, q_pos0=S, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, None, "decode edges")
    assert skipped == ref_skipped
