"""GPU parity of decode over the windowed key cache (atf_decode_pack_k +
atf_decode_kcache, through the C ABI) against the fp64 oracle."""
import math

import numpy as np
import pytest

from parity import check_bf16, log, require_gpu

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


def make_cache(env, k, v, cap, base, pos0=0, pieces=1):
    """Pack k [B,Hkv,S,d] into a cache of capacity cap (in `pieces` appends) and
    copy v into a [B,Hkv,cap,d] buffer (rows past S zero)."""
    torch, oracle, atf, _ = env
    B, Hkv, S, d = k.shape
    kc = torch.empty(atf.atf_decode_kcache_bytes(B, Hkv, cap, d), dtype=torch.uint8, device=k.device)
    bounds = np.linspace(0, S, pieces + 1).astype(int)
    for a0, a1 in zip(bounds[:-1], bounds[1:]):
        if a1 > a0:
            atf.atf_decode_pack_k(k[:, :, a0:a1].contiguous(), kc, k_begin=int(a0), cap=cap, rope_base=base,
                                  pos0=pos0)
    vc = torch.zeros(B, Hkv, cap, d, dtype=v.dtype, device=v.device)
    vc[:, :, :S] = v
    return kc, vc


def run_kcache(env, B, Hq, Hkv, S, cap, d, base, alpha, pos0=0, hf=None, pieces=1):
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=torch.bfloat16, device=dev, high_freq_scale=hf)
    kc, vc = make_cache(env, k, v, cap, base, pos0=pos0, pieces=pieces)
    out, skipped = atf.atf_decode_kcache(q, kc, vc, S=S, rope_base=base, alpha=alpha, pos0=pos0,
                                         return_skipped=True)
    torch.cuda.synchronize()
    return q, k, v, out, skipped


KCACHE = [
    # B, Hq, Hkv, S, cap, d, base, alpha
    (2, 8, 2, 1000, 1024, 128, 1e6, 1.0),
    (1, 7, 1, 300, 320, 128, 1e6, 1.0),
    (3, 28, 4, 4097, 4160, 128, 1e6, 2.0),
    (1, 2, 1, 1, 64, 128, 1e6, 1.0),
    (1, 2, 1, 63, 64, 128, 1e6, 1.0),
    (1, 2, 1, 65, 256, 64, 1e4, 1.0),       # spare capacity
    (1, 4, 4, 5000, 5056, 64, 1e4, 0.5),
    (1, 16, 1, 777, 832, 128, 1e6, 1.0),    # two slabs of 8 query heads
    (1, 3, 1, 2000, 2048, 128, 1e6, math.inf),
    (2, 4, 1, 20000, 20480, 128, 1e6, 1.0),  # many splits
    (1, 3, 1, 3000, 3008, 64, 100.0, 0.3),   # tiny windows: most planes skipped
]


@pytest.mark.parametrize("B,Hq,Hkv,S,cap,d,base,alpha", KCACHE)
def test_kcache_bf16(env, B, Hq, Hkv, S, cap, d, base, alpha):
    torch, oracle, atf, _ = env
    log("case: kcache decode %s" % ((B, Hq, Hkv, S, cap, d, base, alpha),))
    q, k, v, out, skipped = run_kcache(env, B, Hq, Hkv, S, cap, d, base, alpha)
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, q_pos0=S, k_pos0=0)
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, q_pos0=S, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, dense, "kcache %s" % ((B, Hq, Hkv, S, d),))
    assert skipped == ref_skipped == B * Hq * atf.atf_skipped_pair_products(S, d, base, alpha, 1, 1)


def test_kcache_appends_equal_one_write(env):
    """Filling the cache in 5 appends gives the same bytes as one write, so the
    decode result is bit-identical."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(2, 8, 2, 1, 3001, 128, dtype=torch.bfloat16, device=dev)
    kc1, vc = make_cache(env, k, v, 3072, 1e6, pieces=1)
    kc5, _ = make_cache(env, k, v, 3072, 1e6, pieces=5)
    torch.cuda.synchronize()
    # bytes of keys past S are never written: compare the written blocks' key rows only
    blk = kc1.view(2, 2, 3072 // 64, 16, 64, 16)[:, :, :, :, :, :]
    blk5 = kc5.view(2, 2, 3072 // 64, 16, 64, 16)
    nb = 3001 // 64
    assert torch.equal(blk[:, :, :nb], blk5[:, :, :nb])
    r = 3001 % 64
    assert torch.equal(blk[:, :, nb, :, :r], blk5[:, :, nb, :, :r])
    a = atf.atf_decode_kcache(q, kc1, vc, S=3001, rope_base=1e6, alpha=1.0)
    b = atf.atf_decode_kcache(q, kc5, vc, S=3001, rope_base=1e6, alpha=1.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_kcache_grows_with_appends(env):
    """One cache, decoded after each append: every step matches the oracle at
    its own length."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    S_final, cap = 700, 768
    q, k, v = inputs.make_qkv(1, 4, 1, 1, S_final, 128, dtype=torch.bfloat16, device=dev)
    kc = torch.empty(atf.atf_decode_kcache_bytes(1, 1, cap, 128), dtype=torch.uint8, device=dev)
    vc = torch.zeros(1, 1, cap, 128, dtype=torch.bfloat16, device=dev)
    S = 0
    for step in [129, 1, 63, 300, 207]:
        atf.atf_decode_pack_k(k[:, :, S:S + step].contiguous(), kc, k_begin=S, cap=cap, rope_base=1e6)
        vc[:, :, S:S + step] = v[:, :, S:S + step]
        S += step
        out = atf.atf_decode_kcache(q, kc, vc, S=S, rope_base=1e6, alpha=1.0)
        torch.cuda.synchronize()
        ref, _ = oracle.attention(q, k[:, :, :S], v[:, :, :S], base=1e6, alpha=1.0, q_pos0=S, k_pos0=0)
        check_bf16(out.float().cpu().numpy(), ref, None, "kcache S=%d" % S)


def test_kcache_high_frequency_heavy(env):
    torch, oracle, atf, _ = env
    log("case: kcache hf")
    q, k, v, out, skipped = run_kcache(env, 1, 7, 1, 3000, 3008, 128, 1e6, 0.5, hf=1.5)
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=0.5, q_pos0=3000, k_pos0=0)
    dense, _ = oracle.attention(q, k, v, base=1e6, alpha=math.inf, q_pos0=3000, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, dense, "kcache hf", structured=True)
    assert skipped == ref_skipped


@pytest.mark.parametrize("pos0", [1 << 20, 1 << 24])
def test_kcache_position_shift(env, pos0):
    torch, oracle, atf, _ = env
    log("case: kcache pos0=%d" % pos0)
    q, k, v, out, skipped = run_kcache(env, 2, 7, 1, 2500, 2560, 128, 1e6, 1.0, pos0=pos0)
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, q_pos0=pos0 + 2500, k_pos0=pos0)
    check_bf16(out.float().cpu().numpy(), ref, None, "kcache pos0=%d" % pos0)
    assert skipped == ref_skipped


def test_kcache_matches_standard_decode(env):
    """Same query and cache through atf_decode and atf_decode_kcache."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(2, 28, 4, 1, 9000, 128, dtype=torch.bfloat16, device=dev)
    kc, vc = make_cache(env, k, v, 9024, 1e6)
    a = atf.atf_decode(q, k, v, rope_base=1e6, alpha=1.0)
    b = atf.atf_decode_kcache(q, kc, vc, S=9000, rope_base=1e6, alpha=1.0)
    torch.cuda.synchronize()
    check_bf16(b.float().cpu().numpy(), a.float().cpu().numpy(), None, "kcache vs standard")


def test_kcache_workload_full(env):
    """B=8 sequences, query at 262144 after a 262144-key cache, Hq=28, Hkv=4,
    d=128, base 1e6, alpha 1 -- every one of the 224 query rows vs the oracle."""
    torch, oracle, atf, _ = env
    log("case: kcache decode workload S=262144 (all 224 rows)")
    q, k, v, out, skipped = run_kcache(env, 8, 28, 4, 262144, 262144, 128, 1e6, 1.0)
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, q_pos0=262144, k_pos0=0)
    dense, _ = oracle.attention(q, k, v, base=1e6, alpha=math.inf, q_pos0=262144, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, dense, "kcache 256K")
    assert skipped == ref_skipped


STEP = [
    # B, Hq, Hkv, S, cap, d, base, alpha
    (8, 28, 4, 20000, 20032, 128, 1e6, 1.0),
    (2, 7, 1, 4097, 4160, 128, 1e6, 2.0),
    (1, 4, 2, 1, 64, 64, 1e4, 1.0),
    (1, 8, 2, 3001, 3008, 256, 1e6, 1.0),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,cap,d,base,alpha", STEP)
def test_kcache_step_append_then_decode(env, B, Hq, Hkv, S, cap, d, base, alpha):
    """One serving step: the caches hold S - 1 tokens, the step appends token
    S - 1 (its key rotated into the planes, its value row) with one
    atf_decode_append_kv call of n = 1, then decodes the query at S over S
    keys.  Checked against the oracle, and bit for bit against the decode over
    caches written in one go."""
    torch, oracle, atf, inputs = env
    log("case: kcache append-then-decode %s" % ((B, Hq, Hkv, S, cap, d, base, alpha),))
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=torch.bfloat16, device=dev)
    kc = torch.empty(atf.atf_decode_kcache_bytes(B, Hkv, cap, d), dtype=torch.uint8, device=dev)
    vc = torch.zeros(B, Hkv, cap, d, dtype=torch.bfloat16, device=dev)
    if S > 1:
        atf.atf_decode_append_kv(k[:, :, :S - 1].contiguous(), v[:, :, :S - 1].contiguous(), kc, vc, k_begin=0,
                                 cap=cap, rope_base=base)
    atf.atf_decode_append_kv(k[:, :, S - 1:].contiguous(), v[:, :, S - 1:].contiguous(), kc, vc, k_begin=S - 1,
                             cap=cap, rope_base=base)
    out, skipped = atf.atf_decode_kcache(q, kc, vc, S=S, rope_base=base, alpha=alpha, return_skipped=True)
    kc1, vc1 = make_cache(env, k, v, cap, base)
    out1 = atf.atf_decode_kcache(q, kc1, vc1, S=S, rope_base=base, alpha=alpha)
    torch.cuda.synchronize()
    assert torch.equal(vc[:, :, :S], v), "appended value rows"
    assert torch.equal(out, out1), "append-then-decode differs from the decode over a cache written in one go"
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, q_pos0=S, k_pos0=0)
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, q_pos0=S, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, dense, "kcache step %s" % ((B, Hq, Hkv, S, d),))
    assert skipped == ref_skipped == B * Hq * atf.atf_skipped_pair_products(S, d, base, alpha, 1, 1)
