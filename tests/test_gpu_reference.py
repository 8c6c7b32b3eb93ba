"""GPU parity of the online softmax's reference moves (through the C ABI)
against the fp64 oracle.

With iid N(0,1) inputs the softmax reference is set by the first block and
almost never moves again, so the rescale paths (O and l multiplied by
2^(m_old - m_new), the block's probabilities redone) would go untested.  Two
structured inputs force them, using the slowest rotary pair (p = P-1, whose
window is unbounded, so it is kept at every distance):

* ramp: q's pair-(P-1) component is (a, 0) for every query and key j's is
  (c * floor(j / 64), 0), so the logits step up by a*c/sqrt(d) every 64 keys
  (several log2 units) and the reference moves many times along each row.
  The stepped values are exact in bf16 and the pair's rotation over these
  distances is below bf16 resolution, so the step adds no rounding error:
  the usual bf16 tolerance holds.
* spike: one key's pair-(P-1) component is (200, 0) against a query component
  of (8, 0), a logit about 200 log2 units above the rest.  Its probability
  overflows fp32 unless the reference moves before P.V; queries that see it
  must return that key's value.
"""
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


def slow_pair_dims(d):
    """Dims of pair P-1 in the half-split layout: (x, y)."""
    P = d // 2
    return P - 1, d - 1


def ramp(q, k, a, c):
    """Step the logits up every 64 keys through pair P-1 (in place)."""
    x, y = slow_pair_dims(q.shape[-1])
    q[..., x] = a
    q[..., y] = 0
    steps = (np.arange(k.shape[2]) // 64).astype(np.float32) * c
    k[..., x] = k.new_tensor(steps)
    k[..., y] = 0


def spike(q, k, j, qa=8.0, kc=200.0):
    """One key j with a logit about 200 log2 units above the rest (in place)."""
    x, y = slow_pair_dims(q.shape[-1])
    q[..., x] = qa
    q[..., y] = 0
    k[..., x] = 0
    k[..., y] = 0
    k[:, :, j, x] = kc


PREFILL = [
    # d, causal, Hq, Hkv, S, a, c
    (128, True, 2, 1, 1200, 4.0, 8.0),
    (128, False, 2, 1, 1000, 4.0, 8.0),
    (256, True, 2, 1, 1100, 8.0, 8.0),
]


@pytest.mark.parametrize("d,causal,Hq,Hkv,S,a,c", PREFILL)
def test_prefill_reference_moves(env, d, causal, Hq, Hkv, S, a, c):
    torch, oracle, atf, inputs = env
    log("case: prefill ramp d=%d causal=%d S=%d" % (d, causal, S))
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(1, Hq, Hkv, S, S, d, dtype=torch.bfloat16, device=dev)
    ramp(q, k, a, c)
    out, skipped = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0, causal=causal, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, causal=causal)
    check_bf16(out.float().cpu().numpy(), ref, None, "prefill ramp d=%d causal=%d" % (d, causal))
    assert skipped == ref_skipped


@pytest.mark.parametrize("d,causal,S,j", [(128, True, 1200, 700), (128, False, 1000, 613), (256, True, 1100, 700)])
def test_prefill_score_spike(env, d, causal, S, j):
    torch, oracle, atf, inputs = env
    log("case: prefill spike d=%d causal=%d S=%d j=%d" % (d, causal, S, j))
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(1, 2, 1, S, S, d, dtype=torch.bfloat16, device=dev)
    spike(q, k, j)
    out, skipped = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0, causal=causal, return_skipped=True)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, causal=causal)
    check_bf16(got, ref, None, "prefill spike d=%d causal=%d" % (d, causal))
    assert skipped == ref_skipped
    # every query that sees key j returns its value row, to one bf16 ulp (the
    # row sum adds the fp32 probability, P.V its bf16 rounding)
    first = j if causal else 0
    vj = v[0, 0, j].float().cpu().numpy()
    assert np.all(np.abs(got[0, :, first:] - vj) <= np.abs(vj) * 2.0 ** -7 + 1e-6)


@pytest.mark.parametrize("layout", ["standard", "kcache"])
def test_decode_reference_moves(env, layout):
    torch, oracle, atf, inputs = env
    B, Hq, Hkv, S, d = 2, 8, 2, 3000, 128
    log("case: decode ramp %s S=%d" % (layout, S))
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=torch.bfloat16, device=dev)
    ramp(q, k, 4.0, 8.0)
    if layout == "standard":
        out, skipped = atf.atf_decode(q, k, v, rope_base=1e6, alpha=1.0, return_skipped=True)
    else:
        cap = 3008
        kc = torch.empty(atf.atf_decode_kcache_bytes(B, Hkv, cap, d), dtype=torch.uint8, device=dev)
        atf.atf_decode_pack_k(k, kc, k_begin=0, cap=cap, rope_base=1e6)
        vc = torch.zeros(B, Hkv, cap, d, dtype=v.dtype, device=dev)
        vc[:, :, :S] = v
        out, skipped = atf.atf_decode_kcache(q, kc, vc, S=S, rope_base=1e6, alpha=1.0, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, q_pos0=S, k_pos0=0)
    check_bf16(out.float().cpu().numpy(), ref, None, "decode ramp " + layout)
    assert skipped == ref_skipped


def test_decode_score_spike(env):
    torch, oracle, atf, inputs = env
    B, Hq, Hkv, S, d, j = 1, 4, 1, 2500, 128, 1234
    log("case: decode spike S=%d j=%d" % (S, j))
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(B, Hq, Hkv, 1, S, d, dtype=torch.bfloat16, device=dev)
    spike(q, k, j)
    out, skipped = atf.atf_decode(q, k, v, rope_base=1e6, alpha=1.0, return_skipped=True)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, q_pos0=S, k_pos0=0)
    check_bf16(got, ref, None, "decode spike")
    assert skipped == ref_skipped
    vj = v[0, 0, j].float().cpu().numpy()
    assert np.all(np.abs(got[0, :, 0] - vj) <= np.abs(vj) * 2.0 ** -7 + 1e-6)
