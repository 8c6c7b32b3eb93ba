"""GPU parity of non-causal windowed prefill (every key, windows on |i - j|)
through the C ABI, against the fp64 oracle."""
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


NONCAUSAL = [
    # B, Hq, Hkv, S, d, base, alpha
    (1, 1, 1, 256, 64, 1e4, 1.0),
    (1, 7, 1, 300, 128, 1e6, 1.0),
    (2, 4, 2, 1000, 128, 1e6, 0.5),
    (1, 28, 4, 777, 128, 1e6, 2.0),
    (1, 2, 1, 1, 128, 1e6, 1.0),
    (1, 2, 1, 129, 64, 1e4, 1.0),
    (1, 2, 2, 2048, 128, 1e6, 1.0),
    (1, 4, 1, 700, 128, 1e6, math.inf),
    (1, 3, 1, 600, 64, 100.0, 0.3),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,d,base,alpha", NONCAUSAL)
def test_noncausal_bf16(env, B, Hq, Hkv, S, d, base, alpha):
    torch, oracle, atf, inputs = env
    log("case: non-causal bf16 %s" % ((B, Hq, Hkv, S, d, base, alpha),))
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill(q, k, v, rope_base=base, alpha=alpha, causal=0, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha, causal=False)
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf, causal=False)
    check_bf16(out.float().cpu().numpy(), ref, dense, "non-causal %s" % ((B, Hq, Hkv, S, d),))
    assert skipped == ref_skipped == B * Hq * atf.atf_skipped_pair_products(S, d, base, alpha, 0, 0)


def test_noncausal_high_frequency_heavy(env):
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(1, 4, 1, 900, 900, 128, dtype=torch.bfloat16, device=torch.device("cuda:0"),
                              high_freq_scale=1.5)
    out, skipped = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=0.5, causal=0, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=0.5, causal=False)
    dense, _ = oracle.attention(q, k, v, base=1e6, alpha=math.inf, causal=False)
    assert np.abs(dense - ref).max() > 0.05
    check_bf16(out.float().cpu().numpy(), ref, dense, "non-causal hf", structured=True)
    assert skipped == ref_skipped


def test_noncausal_differs_from_causal(env):
    """The first query sees only itself when causal, every key otherwise."""
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(1, 2, 1, 500, 500, 128, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    a = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0, causal=1)
    b = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0, causal=0)
    torch.cuda.synchronize()
    assert (a[:, :, 0] - b[:, :, 0]).abs().max().item() > 0.1


@pytest.mark.parametrize("Sq,Sk", [(100, 1000), (1, 777), (257, 5000)])
def test_noncausal_chunk(env, Sq, Sk):
    """A non-causal chunk sees the keys after each query too (prefix + chunk)."""
    torch, oracle, atf, inputs = env
    log("case: non-causal chunk Sq=%d Sk=%d" % (Sq, Sk))
    q, k, v = inputs.make_qkv(1, 7, 1, Sq, Sk, 128, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill_chunk(q, k, v, rope_base=1e6, alpha=1.0, causal=0, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, causal=False, q_pos0=Sk - Sq, k_pos0=0)
    dense, _ = oracle.attention(q, k, v, base=1e6, alpha=math.inf, causal=False, q_pos0=Sk - Sq, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, dense, "non-causal chunk")
    assert skipped == ref_skipped


@pytest.mark.parametrize("B,Hq,Hkv,S,d", [(1, 1, 1, 256, 64), (2, 4, 2, 333, 128)])
def test_noncausal_fp32(env, B, Hq, Hkv, S, d):
    torch, oracle, atf, inputs = env
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=torch.float32, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill(q, k, v, rope_base=1e4, alpha=1.0, causal=0, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e4, alpha=1.0, causal=False)
    check_f32(out.cpu().numpy(), ref, "non-causal fp32")
    assert skipped == ref_skipped


def test_noncausal_workload_sampled(env):
    """S=32768 at the benchmark heads, sampled rows (first, last, seeded)."""
    torch, oracle, atf, inputs = env
    from rope_frequency_windowed_amd.inputs import sample_rows
    B, Hq, Hkv, S, d = 1, 28, 4, 32768, 128
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0, causal=0, return_skipped=True)
    torch.cuda.synchronize()
    assert skipped == B * Hq * atf.atf_skipped_pair_products(S, d, 1e6, 1.0, 0, 0)
    rows = np.array([(0, h, int(i)) for h in range(0, Hq, 4) for i in sample_rows(S, 4, seed=h)], dtype=np.int64)
    sel = torch.as_tensor(rows, device=q.device)
    qrows = q[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    got = out[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    kk, vv = k.float().cpu().numpy(), v.float().cpu().numpy()
    ref, _ = oracle.attention(qrows, kk, vv, base=1e6, alpha=1.0, causal=False, rows=rows, q_shape=(B, Hq, S, d))
    dense, _ = oracle.attention(qrows, kk, vv, base=1e6, alpha=math.inf, causal=False, rows=rows,
                                q_shape=(B, Hq, S, d))
    check_bf16(got, ref, dense, "non-causal 32K")
