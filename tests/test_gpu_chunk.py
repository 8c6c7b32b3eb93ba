"""GPU parity of chunked prefill (queries after a cached prefix) against the
fp64 oracle, through the C ABI (atf_prefill_chunk)."""
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


def chunk_closed_form(atf, Sq, Sk, d, base, alpha):
    """Per-head dropped terms: F(Sk-1) - F(Sk-Sq-1), F(T) = sum_p n(n+1)/2 with
    n = max(0, T - W_p) (pinned against the oracle's enumeration on the CPU)."""
    W = atf.atf_window_table(d, base, alpha)

    def F(T):
        tot = 0
        for w in W:
            if int(w) == atf.W_INF:
                continue
            n = max(0, T - int(w))
            tot += n * (n + 1) // 2
        return tot
    return F(Sk - 1) - F(Sk - Sq - 1)


def run_chunk(env, B, Hq, Hkv, Sq, Sk, d, base, alpha, dtype, pos0=0, hf=None):
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, Sq, Sk, d, dtype=dtype, device=dev, high_freq_scale=hf)
    out, skipped = atf.atf_prefill_chunk(q, k, v, rope_base=base, alpha=alpha, pos0=pos0, return_skipped=True)
    torch.cuda.synchronize()
    return q, k, v, out, skipped


CHUNK_BF16 = [
    # B, Hq, Hkv, Sq, Sk, d, base, alpha
    (1, 4, 2, 100, 1000, 128, 1e6, 1.0),    # ragged chunk after a ragged prefix
    (1, 7, 1, 1, 777, 128, 1e6, 1.0),       # one query (decode-like, self key included)
    (2, 4, 4, 333, 333, 64, 1e4, 0.5),      # no prefix: plain prefill
    (1, 28, 4, 257, 5000, 128, 1e6, 2.0),   # benchmark head layout
    (1, 2, 1, 64, 4096, 128, 1e6, 1.0),     # one query tile, long prefix
    (1, 3, 1, 300, 2000, 64, 100.0, 0.3),   # tiny windows: most pairs cut
    (1, 2, 1, 513, 1024, 128, 1e6, math.inf),  # no window
]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d,base,alpha", CHUNK_BF16)
def test_chunk_bf16(env, B, Hq, Hkv, Sq, Sk, d, base, alpha):
    torch, oracle, atf, _ = env
    log("case: chunk bf16 %s" % ((B, Hq, Hkv, Sq, Sk, d, base, alpha),))
    q, k, v, out, skipped = run_chunk(env, B, Hq, Hkv, Sq, Sk, d, base, alpha, torch.bfloat16)
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, q_pos0=Sk - Sq, k_pos0=0)
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, q_pos0=Sk - Sq, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, dense, "chunk %s" % ((B, Hq, Hkv, Sq, Sk, d),))
    assert skipped == ref_skipped == B * Hq * chunk_closed_form(atf, Sq, Sk, d, base, alpha)


def test_chunk_high_frequency_heavy(env):
    torch, oracle, atf, _ = env
    log("case: chunk bf16 high-frequency-heavy")
    q, k, v, out, skipped = run_chunk(env, 1, 4, 1, 200, 1500, 128, 1e6, 0.5, torch.bfloat16, hf=1.5)
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=0.5, q_pos0=1300, k_pos0=0)
    dense, _ = oracle.attention(q, k, v, base=1e6, alpha=math.inf, q_pos0=1300, k_pos0=0)
    assert np.abs(dense - ref).max() > 0.05
    check_bf16(out.float().cpu().numpy(), ref, dense, "chunk hf", structured=True)
    assert skipped == ref_skipped


@pytest.mark.parametrize("pos0", [1 << 20, 1 << 24])
def test_chunk_position_shift(env, pos0):
    torch, oracle, atf, _ = env
    log("case: chunk pos0=%d" % pos0)
    q, k, v, out, skipped = run_chunk(env, 1, 2, 1, 150, 700, 128, 1e6, 1.0, torch.bfloat16, pos0=pos0)
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, q_pos0=pos0 + 550, k_pos0=pos0)
    check_bf16(out.float().cpu().numpy(), ref, None, "chunk pos0=%d" % pos0)
    assert skipped == ref_skipped


def test_chunk_without_prefix_is_prefill(env):
    """Sq == Sk: given the minimum workspace (no key split), atf_prefill_chunk
    and atf_prefill agree bit for bit; with the split they agree to rounding."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(1, 4, 2, 700, 700, 128, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(atf.atf_prefill_workspace_bytes(1, 2, 700, 128, atf.ATF_BF16), dtype=torch.uint8, device=dev)
    a = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0)
    b = atf.atf_prefill_chunk(q, k, v, rope_base=1e6, alpha=1.0, ws=ws)
    c = atf.atf_prefill_chunk(q, k, v, rope_base=1e6, alpha=1.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    check_bf16(c.float().cpu().numpy(), a.float().cpu().numpy(), None, "split chunk vs prefill")


def test_chunk_matches_tail_of_full_prefill(env):
    """The chunk's rows agree with the last Sq rows of the full prefill over
    the Sk tokens (same math, different tiling)."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    Sq, Sk = 300, 1100
    q, k, v = inputs.make_qkv(1, 4, 1, Sk, Sk, 128, dtype=torch.bfloat16, device=dev)
    full = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0)
    part = atf.atf_prefill_chunk(q[:, :, Sk - Sq:].contiguous(), k, v, rope_base=1e6, alpha=1.0)
    torch.cuda.synchronize()
    check_bf16(part.float().cpu().numpy(), full[:, :, Sk - Sq:].float().cpu().numpy(), None, "tail")


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d", [(1, 4, 2, 37, 300, 64), (2, 7, 1, 100, 1000, 128)])
def test_chunk_fp32(env, B, Hq, Hkv, Sq, Sk, d):
    torch, oracle, atf, _ = env
    log("case: chunk fp32 %s" % ((B, Hq, Hkv, Sq, Sk, d),))
    q, k, v, out, skipped = run_chunk(env, B, Hq, Hkv, Sq, Sk, d, 1e6, 1.0, torch.float32)
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, q_pos0=Sk - Sq, k_pos0=0)
    check_f32(out.cpu().numpy(), ref, "chunk fp32")
    assert skipped == ref_skipped


def test_chunk_long_prefix_sampled(env):
    """A 4096-token chunk after a 126976-token prefix (Sk = 131072), benchmark
    heads, on sampled rows plus the exact dropped-term count."""
    torch, oracle, atf, _ = env
    from rope_frequency_windowed_amd.inputs import sample_rows
    B, Hq, Hkv, Sq, Sk, d, base, alpha = 1, 28, 4, 4096, 131072, 128, 1e6, 1.0
    log("case: chunk Sq=%d Sk=%d" % (Sq, Sk))
    q, k, v, out, skipped = run_chunk(env, B, Hq, Hkv, Sq, Sk, d, base, alpha, torch.bfloat16)
    assert skipped == B * Hq * chunk_closed_form(atf, Sq, Sk, d, base, alpha)
    rows = np.array([(0, h, int(i)) for h in range(0, Hq, 3) for i in sample_rows(Sq, 4, seed=h)],
                    dtype=np.int64)
    sel = torch.as_tensor(rows, device=q.device)
    qrows = q[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    got = out[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    kk, vv = k.float().cpu().numpy(), v.float().cpu().numpy()
    ref, _ = oracle.attention(qrows, kk, vv, base=base, alpha=alpha, q_pos0=Sk - Sq, k_pos0=0,
                              rows=rows, q_shape=(B, Hq, Sq, d))
    dense, _ = oracle.attention(qrows, kk, vv, base=base, alpha=math.inf, q_pos0=Sk - Sq, k_pos0=0,
                                rows=rows, q_shape=(B, Hq, Sq, d))
    check_bf16(got, ref, dense, "chunk long prefix")


@pytest.mark.parametrize("d,causal", [(64, 1), (128, 1), (128, 0), (256, 1), (256, 0)])
def test_chunk_key_split_matches_unsplit(env, d, causal):
    """A short chunk over a long prefix: with the larger workspace the key
    range of each query tile is split over workgroups and merged by the
    combine kernel; with the minimum workspace it is not.  Both against the
    oracle, with the same dropped-term count."""
    torch, oracle, atf, inputs = env
    B, Hq, Hkv, Sq, Sk, base, alpha = 1, 4, 2, 40, 3000, 1e6, 1.0
    log("case: chunk key split d=%d causal=%d" % (d, causal))
    dev = torch.device("cuda:0")
    small = atf.atf_prefill_workspace_bytes(B, Hkv, Sk, d, atf.ATF_BF16)
    big = atf.atf_prefill_chunk_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, atf.ATF_BF16)
    assert big > small  # the planner splits this shape
    q, k, v = inputs.make_qkv(B, Hq, Hkv, Sq, Sk, d, dtype=torch.bfloat16, device=dev)
    outs = []
    for nb in (small, big):
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        outs.append(atf.atf_prefill_chunk(q, k, v, rope_base=base, alpha=alpha, causal=causal, ws=ws,
                                          return_skipped=True))
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, causal=bool(causal), q_pos0=Sk - Sq,
                                        k_pos0=0)
    for (out, skipped), name in zip(outs, ("unsplit", "split")):
        check_bf16(out.float().cpu().numpy(), ref, None, "chunk %s d=%d causal=%d" % (name, d, causal))
        assert skipped == ref_skipped


@pytest.mark.parametrize("d", [128, 256])
def test_chunk_short_after_long_prefix(env, d):
    """16 queries after 32752 cached tokens: the planner's widest splits
    (64 per query tile), every row against the oracle."""
    torch, oracle, atf, _ = env
    B, Hq, Hkv, Sq, Sk, base, alpha = 1, 4, 1, 16, 32768, 1e6, 1.0
    log("case: chunk Sq=%d Sk=%d d=%d" % (Sq, Sk, d))
    q, k, v, out, skipped = run_chunk(env, B, Hq, Hkv, Sq, Sk, d, base, alpha, torch.bfloat16)
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, q_pos0=Sk - Sq, k_pos0=0)
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, q_pos0=Sk - Sq, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, dense, "chunk short after long prefix d=%d" % d)
    assert skipped == ref_skipped == B * Hq * chunk_closed_form(atf, Sq, Sk, d, base, alpha)


@pytest.mark.parametrize("d,Hq,Hkv,rows", [(128, 8, 1, 32), (256, 16, 2, 16)])
def test_chunk_head_packed_matches_unpacked(env, d, Hq, Hkv, rows):
    """A chunk of one wave's rows runs head packed (one wave per query head of
    a kv group); a 1024-query chunk ending at the same token runs unpacked.
    The shared rows form the same wave blocks over the same key tiles, so
    they agree bit for bit (minimum workspace: no key split)."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    Sk, base, alpha = 3000, 1e6, 1.0
    log("case: chunk head packed vs unpacked d=%d" % d)
    q, k, v = inputs.make_qkv(1, Hq, Hkv, 1024, Sk, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(atf.atf_prefill_workspace_bytes(1, Hkv, Sk, d, atf.ATF_BF16), dtype=torch.uint8, device=dev)
    full = atf.atf_prefill_chunk(q, k, v, rope_base=base, alpha=alpha, ws=ws)
    tail = atf.atf_prefill_chunk(q[:, :, 1024 - rows:].contiguous(), k, v, rope_base=base, alpha=alpha, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(tail, full[:, :, 1024 - rows:])


@pytest.mark.parametrize("Hq,Hkv,Sq,d", [(16, 1, 40, 128), (12, 1, 33, 128), (24, 2, 20, 256), (5, 1, 7, 64)])
def test_chunk_head_packed_slabs(env, Hq, Hkv, Sq, d):
    """Head-packed chunks with more heads per kv head than waves (two slabs,
    the second partly idle) or fewer (idle waves), against the oracle."""
    torch, oracle, atf, _ = env
    Sk, base, alpha = 2500, 1e6, 1.0
    log("case: chunk head packed Hq=%d Hkv=%d Sq=%d d=%d" % (Hq, Hkv, Sq, d))
    q, k, v, out, skipped = run_chunk(env, 1, Hq, Hkv, Sq, Sk, d, base, alpha, torch.bfloat16)
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, q_pos0=Sk - Sq, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, None, "chunk head packed %s" % ((Hq, Hkv, Sq, d),))
    assert skipped == ref_skipped


@pytest.mark.parametrize("Hq,Hkv,Sq,Sk,causal", [
    (28, 4, 16, 9000, 1), (7, 1, 5, 3001, 1), (16, 1, 1, 2000, 1), (28, 4, 16, 5000, 0), (8, 2, 9, 300, 1)])
def test_chunk_narrow_d128(env, Hq, Hkv, Sq, Sk, causal):
    """d = 128 chunks of at most 16 queries run head packed on the 16x16x32
    kernel (16-query waves), with the key split; against the oracle."""
    torch, oracle, atf, _ = env
    base, alpha = 1e6, 1.0
    log("case: chunk narrow d=128 %s" % ((Hq, Hkv, Sq, Sk, causal),))
    dev = torch.device("cuda:0")
    from rope_frequency_windowed_amd import inputs
    q, k, v = inputs.make_qkv(1, Hq, Hkv, Sq, Sk, 128, dtype=torch.bfloat16, device=dev)
    out, skipped = atf.atf_prefill_chunk(q, k, v, rope_base=base, alpha=alpha, causal=causal, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, causal=bool(causal), q_pos0=Sk - Sq,
                                        k_pos0=0)
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, causal=bool(causal), q_pos0=Sk - Sq, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, dense, "chunk narrow %s" % ((Hq, Hkv, Sq, Sk, causal),))
    assert skipped == ref_skipped


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d", [(3, 8, 2, 20, 2000, 128), (2, 14, 2, 8, 3000, 128),
                                              (2, 6, 3, 40, 1500, 64), (2, 16, 2, 10, 1200, 256)])
def test_chunk_split_packed_batch(env, B, Hq, Hkv, Sq, Sk, d):
    """Key split with head-packed (and, for 8 queries at d = 128, narrow) work
    items over several sequences: the partials and work items index by batch."""
    torch, oracle, atf, _ = env
    base, alpha = 1e6, 1.0
    log("case: chunk split packed batch %s" % ((B, Hq, Hkv, Sq, Sk, d),))
    assert atf.atf_prefill_chunk_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, atf.ATF_BF16) > \
        atf.atf_prefill_workspace_bytes(B, Hkv, Sk, d, atf.ATF_BF16)
    q, k, v, out, skipped = run_chunk(env, B, Hq, Hkv, Sq, Sk, d, base, alpha, torch.bfloat16)
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, q_pos0=Sk - Sq, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, None, "chunk split packed batch %s" % ((B, Hq, Hkv, Sq, Sk, d),))
    assert skipped == ref_skipped == B * Hq * chunk_closed_form(atf, Sq, Sk, d, base, alpha)


def test_chunk_full_round_split(env):
    """270 query-tile workgroups (just over one round of 256) after a prefix of
    more than three chunks: the planner splits the key range in two so the
    rounds come out full; every row against the oracle."""
    torch, oracle, atf, _ = env
    B, Hq, Hkv, Sq, Sk, d, base, alpha = 3, 90, 90, 100, 520, 64, 1e4, 1.0
    log("case: chunk full-round split %s" % ((B, Hq, Hkv, Sq, Sk, d),))
    assert atf.atf_prefill_chunk_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, atf.ATF_BF16) == \
        atf.atf_prefill_workspace_bytes(B, Hkv, Sk, d, atf.ATF_BF16) + B * Hq * Sq * 2 * (d + 2) * 4
    q, k, v, out, skipped = run_chunk(env, B, Hq, Hkv, Sq, Sk, d, base, alpha, torch.bfloat16)
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, q_pos0=Sk - Sq, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, None, "chunk full-round split")
    assert skipped == ref_skipped == B * Hq * chunk_closed_form(atf, Sq, Sk, d, base, alpha)


@pytest.mark.parametrize("d,Sq,layout,pos0", [(128, 16, "gptj", 0), (128, 5, "gptj", 1 << 20),
                                              (256, 16, "gptj", 12345), (256, 40, "neox", 1 << 22)])
def test_chunk_split_rotated_queries(env, d, Sq, layout, pos0):
    """Key-split chunks on 16-query waves rotate their queries once, in a pass
    of their own, for all splits: both rotary layouts and shifted positions
    against the oracle, with the exact dropped-term count."""
    torch, oracle, atf, inputs = env
    B, Hq, Hkv, Sk, base, alpha = 2, 8, 2, 2500, 1e6, 1.0
    log("case: chunk split rotated queries d=%d Sq=%d %s pos0=%d" % (d, Sq, layout, pos0))
    dev = torch.device("cuda:0")
    assert atf.atf_prefill_chunk_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, atf.ATF_BF16) > \
        atf.atf_prefill_workspace_bytes(B, Hkv, Sk, d, atf.ATF_BF16)
    q, k, v = inputs.make_qkv(B, Hq, Hkv, Sq, Sk, d, dtype=torch.bfloat16, device=dev)
    out, skipped = atf.atf_prefill_chunk(q, k, v, rope_base=base, alpha=alpha, pos0=pos0, rope_layout=layout,
                                         return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, q_pos0=pos0 + Sk - Sq, k_pos0=pos0,
                                        layout=layout)
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, q_pos0=pos0 + Sk - Sq, k_pos0=pos0,
                                layout=layout)
    check_bf16(out.float().cpu().numpy(), ref, dense, "chunk split rotated queries d=%d Sq=%d %s" % (d, Sq, layout))
    assert skipped == ref_skipped == B * Hq * chunk_closed_form(atf, Sq, Sk, d, base, alpha)
