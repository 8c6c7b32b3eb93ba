"""GPU parity of chunked prefill over a kept prefill cache
(atf_prefill_cache_append + atf_prefill_chunk_cached, through the C ABI):
bit for bit against atf_prefill_chunk over the same keys, and against the
fp64 oracle."""
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


def new_cache(torch, atf, B, Hkv, cap, d, dev):
    # filled with a NaN pattern: every byte the attention reads must have been written
    return torch.full((atf.atf_prefill_cache_bytes(B, Hkv, cap, d),), 0xFF, dtype=torch.uint8, device=dev)


@pytest.mark.parametrize("d,Hq,Hkv", [(128, 28, 4), (64, 4, 2), (256, 8, 2)])
def test_cache_appends_match_chunk(env, d, Hq, Hkv):
    """A serving loop: ragged chunks appended one after another (appends start
    and end inside tiles); after each, the chunk's queries attend over the
    cache.  Each step equals atf_prefill_chunk over the same keys bit for bit
    (same split plan); the last step is checked against the oracle."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    B, cap, base, alpha = 1, 3000, 1e6, 1.0
    chunks = [1000, 37, 1, 600, 100]
    S = sum(chunks)
    log("case: prefill cache appends d=%d chunks %s" % (d, chunks))
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=torch.bfloat16, device=dev)
    cache = new_cache(torch, atf, B, Hkv, cap, d, dev)
    end = 0
    for n in chunks:
        atf.atf_prefill_cache_append(k[:, :, end:end + n].contiguous(), v[:, :, end:end + n].contiguous(), cache,
                                     k_begin=end, cap=cap, rope_base=base)
        end += n
        qc = q[:, :, end - n:end].contiguous()
        got, sk_got = atf.atf_prefill_chunk_cached(qc, cache, Hkv=Hkv, Sk=end, cap=cap, rope_base=base, alpha=alpha,
                                                   return_skipped=True)
        want, sk_want = atf.atf_prefill_chunk(qc, k[:, :, :end].contiguous(), v[:, :, :end].contiguous(),
                                              rope_base=base, alpha=alpha, return_skipped=True)
        torch.cuda.synchronize()
        assert torch.equal(got, want), "step Sk=%d differs from atf_prefill_chunk" % end
        assert sk_got == sk_want
    ref, ref_skipped = oracle.attention(qc, k, v, base=base, alpha=alpha, q_pos0=S - chunks[-1], k_pos0=0)
    check_bf16(got.float().cpu().numpy(), ref, None, "cache last chunk d=%d" % d)
    assert sk_got == ref_skipped


@pytest.mark.parametrize("causal", [1, 0])
def test_cache_attend_below_filled_length(env, causal):
    """Sk below the cache's filled length: the keys past Sk (real values, not
    cleared) stay out of the softmax, causal or not."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, cap, base, alpha = 1, 8, 2, 128, 2048, 1e6, 1.0
    filled, Sk, Sq = 1700, 1203, 70
    log("case: prefill cache Sk=%d < filled=%d causal=%d" % (Sk, filled, causal))
    q, k, v = inputs.make_qkv(B, Hq, Hkv, Sq, filled, d, dtype=torch.bfloat16, device=dev)
    cache = new_cache(torch, atf, B, Hkv, cap, d, dev)
    atf.atf_prefill_cache_append(k, v, cache, k_begin=0, cap=cap, rope_base=base)
    got = atf.atf_prefill_chunk_cached(q, cache, Hkv=Hkv, Sk=Sk, cap=cap, rope_base=base, alpha=alpha, causal=causal)
    want = atf.atf_prefill_chunk(q, k[:, :, :Sk].contiguous(), v[:, :, :Sk].contiguous(), rope_base=base,
                                 alpha=alpha, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    ref, _ = oracle.attention(q, k[:, :, :Sk], v[:, :, :Sk], base=base, alpha=alpha, causal=bool(causal),
                              q_pos0=Sk - Sq, k_pos0=0)
    check_bf16(got.float().cpu().numpy(), ref, None, "cache below filled causal=%d" % causal)


def test_cache_gptj_and_position_shift(env):
    """Interleaved rotary pairs and a shifted start position (pos0 = 2^20)."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, cap, base, alpha, pos0 = 2, 4, 1, 128, 1500, 1e6, 1.0, 1 << 20
    chunks = [700, 300]
    S = sum(chunks)
    log("case: prefill cache gptj pos0=%d" % pos0)
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=torch.bfloat16, device=dev)
    cache = new_cache(torch, atf, B, Hkv, cap, d, dev)
    end = 0
    for n in chunks:
        atf.atf_prefill_cache_append(k[:, :, end:end + n].contiguous(), v[:, :, end:end + n].contiguous(), cache,
                                     k_begin=end, cap=cap, rope_base=base, pos0=pos0, rope_layout="gptj")
        end += n
    qc = q[:, :, S - chunks[-1]:].contiguous()
    got = atf.atf_prefill_chunk_cached(qc, cache, Hkv=Hkv, Sk=S, cap=cap, rope_base=base, alpha=alpha, pos0=pos0,
                                       rope_layout="gptj")
    want = atf.atf_prefill_chunk(qc, k, v, rope_base=base, alpha=alpha, pos0=pos0, rope_layout="gptj")
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    ref, _ = oracle.attention(qc, k, v, base=base, alpha=alpha, q_pos0=pos0 + S - chunks[-1], k_pos0=pos0,
                              layout="gptj")
    check_bf16(got.float().cpu().numpy(), ref, None, "cache gptj")


def test_cache_minimum_scratch_is_unsplit(env):
    """With only the 256-byte scratch the call runs unsplit, and equals the
    unsplit atf_prefill_chunk (minimum workspace) bit for bit."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    B, Hq, Hkv, d, cap, base, alpha, Sq, Sk = 1, 28, 4, 128, 8192, 1e6, 1.0, 16, 8000
    q, k, v = inputs.make_qkv(B, Hq, Hkv, Sq, Sk, d, dtype=torch.bfloat16, device=dev)
    assert atf.atf_prefill_cached_scratch_bytes(B, Hq, Hkv, Sq, Sk, d) > 256
    cache = new_cache(torch, atf, B, Hkv, cap, d, dev)
    atf.atf_prefill_cache_append(k, v, cache, k_begin=0, cap=cap, rope_base=base)
    scratch = torch.empty(256, dtype=torch.uint8, device=dev)
    got = atf.atf_prefill_chunk_cached(q, cache, Hkv=Hkv, Sk=Sk, cap=cap, rope_base=base, alpha=alpha,
                                       scratch=scratch)
    ws = torch.empty(atf.atf_prefill_workspace_bytes(B, Hkv, Sk, d, atf.ATF_BF16), dtype=torch.uint8, device=dev)
    want = atf.atf_prefill_chunk(q, k, v, rope_base=base, alpha=alpha, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
