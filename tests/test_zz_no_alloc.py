"""GPU test of atf_decode_paged_noalloc (the paged decode that allocates
nothing: its scratch is the library's static device array), through the C ABI:
two calls in a row, the second smaller, each bit-identical to
atf_decode_paged with a caller workspace and within the bf16 bound of the
fp64 oracle, with the exact dropped-term count."""
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


def paged_inputs(env, B, Hq, Hkv, lens, d, base, seed):
    torch, _, atf, inputs = env
    dev = torch.device("cuda:0")
    max_len = max(lens)
    max_pages = (max_len + 63) // 64
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, max_len, d, dtype=torch.bfloat16, device=dev,
                              seeds=(1000 + seed, 1001 + seed, 1002 + seed))
    num_pages = B * max_pages + 3
    perm = np.random.default_rng(seed).permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    pt = torch.as_tensor(perm.astype(np.int32), device=dev)
    pb = atf.atf_paged_page_bytes(Hkv, d)
    kpool = torch.zeros(num_pages, Hkv, pb // Hkv, dtype=torch.uint8, device=dev)
    vpool = torch.zeros(num_pages, Hkv, pb // Hkv, dtype=torch.uint8, device=dev)
    atf.atf_paged_write(k, v, kpool, vpool, pt, k_begin=0, rope_base=base)
    sl = torch.as_tensor(np.array(lens, dtype=np.int32), device=dev)
    return q, k, v, kpool, vpool, pt, sl, max_len


CALLS = [
    # B, Hq, Hkv, lens, d, base, alpha: the second call is smaller than the first
    (8, 28, 4, [65536, 40000, 70000, 1, 64, 65, 12345, 30000], 128, 1e6, 1.0),
    (2, 7, 1, [3000, 100], 128, 1e6, 2.0),
]


def test_noalloc_matches_workspace_decode_twice(env):
    torch, oracle, atf, _ = env
    for n, (B, Hq, Hkv, lens, d, base, alpha) in enumerate(CALLS):
        log("case: noalloc paged decode call %d %s" % (n, (B, Hq, Hkv, lens, d, base, alpha)))
        assert atf.atf_decode_paged_workspace_bytes(B, Hq, Hkv, max(lens), d) <= atf.NOALLOC_SCRATCH_BYTES
        q, k, v, kpool, vpool, pt, sl, max_len = paged_inputs(env, B, Hq, Hkv, lens, d, base, seed=n)
        ref_out, ref_sk = atf.atf_decode_paged(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=base,
                                               alpha=alpha, return_skipped=True)
        out, sk = atf.atf_decode_paged_noalloc(q, kpool, vpool, pt, sl, max_len=max_len, rope_base=base,
                                               alpha=alpha, return_skipped=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "call %d: differs from atf_decode_paged" % n
        closed = Hq * sum(atf.atf_skipped_pair_products(S, d, base, alpha, 1, 1) for S in lens)
        assert sk == ref_sk == closed
        # oracle on a few sequences of each call (all of the small one)
        for b in ([0, 3, 6] if B > 2 else range(B)):
            S = lens[b]
            qb, kb, vb = q[b:b + 1], k[b:b + 1, :, :S], v[b:b + 1, :, :S]
            ref, _ = oracle.attention(qb, kb, vb, base=base, alpha=alpha, q_pos0=S, k_pos0=0)
            dense, _ = oracle.attention(qb, kb, vb, base=base, alpha=math.inf, q_pos0=S, k_pos0=0)
            check_bf16(out[b:b + 1].float().cpu().numpy(), ref, dense, "noalloc call %d seq %d" % (n, b))
