"""GPU parity of paged, ragged decode (atf_paged_write + atf_decode_paged,
through the C ABI) against the fp64 oracle, one sequence at a time."""
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


def build_paged(env, B, Hq, Hkv, lens, d, base, pos0=0, spare_pages=5, seed=0, hf=None, max_len=None):
    """Random page table over a shuffled pool; every sequence's first max_len
    tokens written through atf_paged_write (the kernel reads only seq_lens[b])."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    max_len = max(lens) if max_len is None else max_len
    max_pages = (max_len + 63) // 64
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, max_len, d, dtype=torch.bfloat16, device=dev, high_freq_scale=hf)
    num_pages = B * max_pages + spare_pages
    perm = np.random.default_rng(seed).permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    pt = torch.as_tensor(perm.astype(np.int32), device=dev)
    pb = atf.atf_paged_page_bytes(Hkv, d)
    kpool = torch.zeros(num_pages, Hkv, pb // Hkv, dtype=torch.uint8, device=dev)
    vpool = torch.zeros(num_pages, Hkv, pb // Hkv, dtype=torch.uint8, device=dev)
    atf.atf_paged_write(k, v, kpool, vpool, pt, k_begin=0, rope_base=base, pos0=pos0)
    sl = torch.as_tensor(np.array(lens, dtype=np.int32), device=dev)
    return q, k, v, kpool, vpool, pt, sl, max_len


def check_against_oracle(env, q, k, v, out, lens, base, alpha, pos0=0, structured=False, label=""):
    torch, oracle, atf, _ = env
    total_skipped = 0
    for b, S in enumerate(lens):
        qb, kb, vb = q[b:b + 1], k[b:b + 1, :, :S], v[b:b + 1, :, :S]
        ref, sk = oracle.attention(qb, kb, vb, base=base, alpha=alpha, q_pos0=pos0 + S, k_pos0=pos0)
        dense, _ = oracle.attention(qb, kb, vb, base=base, alpha=math.inf, q_pos0=pos0 + S, k_pos0=pos0)
        check_bf16(out[b:b + 1].float().cpu().numpy(), ref, dense, "%s seq %d (S=%d)" % (label, b, S),
                   structured=structured)
        total_skipped += sk
    return total_skipped


PAGED = [
    # B, Hq, Hkv, lens, d, base, alpha
    (3, 8, 2, [1000, 1, 777], 128, 1e6, 1.0),
    (4, 7, 1, [300, 64, 65, 2049], 128, 1e6, 1.0),
    (2, 28, 4, [4097, 4096], 128, 1e6, 2.0),
    (5, 4, 4, [5000, 63, 129, 1024, 3333], 64, 1e4, 0.5),
    (2, 16, 1, [777, 200], 128, 1e6, 1.0),           # two slabs of 8 query heads
    (3, 3, 1, [2000, 500, 1999], 128, 1e6, math.inf),
    (2, 4, 1, [20000, 9000], 128, 1e6, 1.0),         # many splits, some empty for the short one
    (3, 3, 1, [3000, 3001, 17], 64, 100.0, 0.3),     # tiny windows
]


@pytest.mark.parametrize("B,Hq,Hkv,lens,d,base,alpha", PAGED)
def test_paged_bf16(env, B, Hq, Hkv, lens, d, base, alpha):
    torch, oracle, atf, _ = env
    log("case: paged decode %s" % ((B, Hq, Hkv, lens, d, base, alpha),))
    q, k, v, kpool, vpool, pt, sl, max_len = build_paged(env, B, Hq, Hkv, lens, d, base)
    out, skipped = atf.atf_decode_paged(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=base, alpha=alpha,
                                        return_skipped=True)
    torch.cuda.synchronize()
    ref_skipped = check_against_oracle(env, q, k, v, out, lens, base, alpha, label="paged")
    assert skipped == ref_skipped == Hq * sum(atf.atf_skipped_pair_products(S, d, base, alpha, 1, 1) for S in lens)


def test_paged_large_batch(env):
    """150 sequences of seeded random lengths 1..1200: the split ids are mapped
    to sequences 64 at a time, so three scan steps and a sequence straddling
    the first step boundary are exercised; every row against the oracle."""
    torch, oracle, atf, _ = env
    lens = [int(x) for x in np.random.default_rng(150).integers(1, 1201, size=150)]
    B, Hq, Hkv, d, base, alpha = len(lens), 2, 1, 128, 1e6, 1.0
    log("case: paged decode, %d sequences" % B)
    q, k, v, kpool, vpool, pt, sl, max_len = build_paged(env, B, Hq, Hkv, lens, d, base)
    out, skipped = atf.atf_decode_paged(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=base, alpha=alpha,
                                        return_skipped=True)
    torch.cuda.synchronize()
    ref_skipped = check_against_oracle(env, q, k, v, out, lens, base, alpha, label="paged large batch")
    assert skipped == ref_skipped == Hq * sum(atf.atf_skipped_pair_products(S, d, base, alpha, 1, 1) for S in lens)


def test_paged_max_len_above_lengths(env):
    """max_len (planning bound) larger than every length: same answer."""
    torch, oracle, atf, _ = env
    lens = [900, 1200]
    q, k, v, kpool, vpool, pt, sl, max_len = build_paged(env, 2, 4, 2, lens, 128, 1e6, max_len=5000)
    out = atf.atf_decode_paged(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=1e6, alpha=1.0)
    torch.cuda.synchronize()
    check_against_oracle(env, q, k, v, out, lens, 1e6, 1.0, label="paged max_len")


def test_paged_lengths_change_between_calls(env):
    """Same pages, new lengths (device array): no host replanning needed."""
    torch, oracle, atf, _ = env
    q, k, v, kpool, vpool, pt, sl, max_len = build_paged(env, 3, 7, 1, [3000, 3000, 3000], 128, 1e6)
    for lens in ([3000, 10, 2500], [1, 2999, 64]):
        sl.copy_(torch.as_tensor(np.array(lens, dtype=np.int32)))
        out = atf.atf_decode_paged(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=1e6, alpha=1.0)
        torch.cuda.synchronize()
        check_against_oracle(env, q, k, v, out, lens, 1e6, 1.0, label="paged lens %s" % lens)


def test_paged_high_frequency_heavy(env):
    torch, oracle, atf, _ = env
    lens = [3000, 1500]
    q, k, v, kpool, vpool, pt, sl, max_len = build_paged(env, 2, 7, 1, lens, 128, 1e6, hf=1.5)
    out = atf.atf_decode_paged(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=1e6, alpha=0.5)
    torch.cuda.synchronize()
    check_against_oracle(env, q, k, v, out, lens, 1e6, 0.5, structured=True, label="paged hf")


@pytest.mark.parametrize("pos0", [1 << 20, 1 << 24])
def test_paged_position_shift(env, pos0):
    torch, oracle, atf, _ = env
    lens = [2500, 700]
    q, k, v, kpool, vpool, pt, sl, max_len = build_paged(env, 2, 7, 1, lens, 128, 1e6, pos0=pos0)
    out = atf.atf_decode_paged(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=1e6, alpha=1.0, pos0=pos0)
    torch.cuda.synchronize()
    check_against_oracle(env, q, k, v, out, lens, 1e6, 1.0, pos0=pos0, label="paged pos0=%d" % pos0)


def test_paged_matches_contiguous_key_cache(env):
    """Equal lengths: paged decode agrees with atf_decode_kcache on the same data."""
    torch, oracle, atf, _ = env
    lens = [9000, 9000]
    q, k, v, kpool, vpool, pt, sl, max_len = build_paged(env, 2, 28, 4, lens, 128, 1e6)
    cap = 9024
    kc = torch.empty(atf.atf_decode_kcache_bytes(2, 4, cap, 128), dtype=torch.uint8, device=q.device)
    atf.atf_decode_pack_k(k, kc, k_begin=0, cap=cap, rope_base=1e6)
    vc = torch.zeros(2, 4, cap, 128, dtype=torch.bfloat16, device=q.device)
    vc[:, :, :9000] = v
    a = atf.atf_decode_kcache(q, kc, vc, S=9000, rope_base=1e6, alpha=1.0)
    b = atf.atf_decode_paged(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=1e6, alpha=1.0)
    torch.cuda.synchronize()
    check_bf16(b.float().cpu().numpy(), a.float().cpu().numpy(), None, "paged vs contiguous")


def test_paged_workload_ragged(env):
    """Benchmark heads (Hq=28, Hkv=4, d=128, base 1e6, alpha 1), 8 ragged
    sequences up to 262144 tokens, every query row against the oracle."""
    torch, oracle, atf, _ = env
    lens = [262144, 131072, 100000, 65537, 8191, 4096, 64, 1]
    log("case: paged ragged workload %s" % lens)
    q, k, v, kpool, vpool, pt, sl, max_len = build_paged(env, 8, 28, 4, lens, 128, 1e6, spare_pages=0)
    out, skipped = atf.atf_decode_paged(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=1e6, alpha=1.0,
                                        return_skipped=True)
    torch.cuda.synchronize()
    ref_skipped = check_against_oracle(env, q, k, v, out, lens, 1e6, 1.0, label="paged 256K ragged")
    assert skipped == ref_skipped


@pytest.mark.parametrize("B,Hq,Hkv,S,d,base,alpha", [
    (8, 28, 4, 20000, 128, 1e6, 1.0),
    (3, 7, 1, 4097, 128, 1e6, 2.0),
    (2, 4, 2, 1, 64, 1e4, 1.0),
])
def test_paged_step_append_then_decode(env, B, Hq, Hkv, S, d, base, alpha):
    """One serving step over pages: every sequence holds S - 1 tokens, the step
    writes token S - 1 of each (atf_paged_write, n = 1), then decodes the
    queries at S.  Checked against the oracle and bit for bit against the same
    decode over pages written in one go."""
    torch, oracle, atf, inputs = env
    log("case: paged append-then-decode %s" % ((B, Hq, Hkv, S, d, base, alpha),))
    dev = torch.device("cuda:0")
    max_pages = (S + 63) // 64
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=torch.bfloat16, device=dev)
    num_pages = B * max_pages + 2
    perm = np.random.default_rng(3).permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    pt = torch.as_tensor(perm.astype(np.int32), device=dev)
    pb = atf.atf_paged_page_bytes(Hkv, d)
    pools = [torch.zeros(num_pages, Hkv, pb // Hkv, dtype=torch.uint8, device=dev) for _ in range(4)]
    if S > 1:
        atf.atf_paged_write(k[:, :, :S - 1].contiguous(), v[:, :, :S - 1].contiguous(), pools[0], pools[1], pt,
                            k_begin=0, rope_base=base)
    atf.atf_paged_write(k[:, :, S - 1:].contiguous(), v[:, :, S - 1:].contiguous(), pools[0], pools[1], pt,
                        k_begin=S - 1, rope_base=base)
    atf.atf_paged_write(k, v, pools[2], pools[3], pt, k_begin=0, rope_base=base)
    sl = torch.full((B,), S, dtype=torch.int32, device=dev)
    out, skipped = atf.atf_decode_paged(q, pools[0], pools[1], pt, sl, max_len=S, rope_base=base, alpha=alpha,
                                        return_skipped=True)
    out1 = atf.atf_decode_paged(q, pools[2], pools[3], pt, sl, max_len=S, rope_base=base, alpha=alpha)
    torch.cuda.synchronize()
    assert torch.equal(out, out1), "append-then-decode differs from the decode over pages written in one go"
    ref_skipped = check_against_oracle(env, q, k, v, out, [S] * B, base, alpha, label="paged step")
    assert skipped == ref_skipped == B * Hq * atf.atf_skipped_pair_products(S, d, base, alpha, 1, 1)
