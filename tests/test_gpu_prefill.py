"""GPU parity of the prefill path (through the C ABI) against the fp64 oracle."""
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


def run_prefill(env, B, Hq, Hkv, S, d, base, alpha, dtype, pos0=0, hf=None, seeds=None):
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    kw = {} if seeds is None else {"seeds": seeds}
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=dtype, device=dev, high_freq_scale=hf, **kw)
    out, skipped = atf.atf_prefill(q, k, v, rope_base=base, alpha=alpha, pos0=pos0, return_skipped=True)
    torch.cuda.synchronize()
    return q, k, v, out, skipped


def test_small_fp32_config(env):
    """B=1, H=1, S=256, d=64, base 1e4, alpha 1, fp32: max-abs 1e-5, count exact."""
    torch, oracle, atf, _ = env
    log("case: fp32 S=256 d=64")
    q, k, v, out, skipped = run_prefill(env, 1, 1, 1, 256, 64, 1e4, 1.0, torch.float32)
    ref, ref_skipped = oracle.attention(q, k, v, base=1e4, alpha=1.0)
    check_f32(out.cpu().numpy(), ref, "fp32 S=256")
    assert skipped == ref_skipped == 270074


@pytest.mark.parametrize("B,Hq,Hkv,S,d,base,alpha", [
    (1, 2, 1, 333, 64, 1e4, 0.5),
    (1, 4, 2, 1000, 128, 1e6, 1.0),
    (2, 3, 3, 70, 128, 1e6, 2.0),
    (1, 1, 1, 1, 64, 1e4, 1.0),
])
def test_fp32_shapes(env, B, Hq, Hkv, S, d, base, alpha):
    torch, oracle, atf, _ = env
    log("case: fp32 %s" % ((B, Hq, Hkv, S, d, base, alpha),))
    q, k, v, out, skipped = run_prefill(env, B, Hq, Hkv, S, d, base, alpha, torch.float32)
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha)
    check_f32(out.cpu().numpy(), ref, "fp32")
    assert skipped == ref_skipped


SMALL_BF16 = [
    # B, Hq, Hkv, S, d, base, alpha
    (1, 1, 1, 256, 64, 1e4, 1.0),       # the small workload in bf16
    (1, 7, 1, 300, 128, 1e6, 1.0),      # one GQA group, ragged tail
    (2, 4, 2, 1000, 128, 1e6, 0.5),     # several tiles, ragged
    (1, 28, 4, 777, 128, 1e6, 2.0),     # the benchmark head layout
    (1, 2, 1, 1, 128, 1e6, 1.0),        # single token
    (1, 2, 1, 5, 128, 1e6, 1.0),        # S < W_0: nothing cut
    (1, 2, 1, 64, 128, 1e6, 1.0),       # exactly one key tile
    (1, 2, 1, 129, 64, 1e4, 1.0),       # one past a query tile
    (1, 2, 2, 2048, 128, 1e6, 1.0),
    (1, 4, 1, 700, 128, 1e6, math.inf),  # no window at all
    (1, 3, 1, 600, 64, 100.0, 0.3),     # tiny windows: most pairs cut near the diagonal
]


@pytest.mark.parametrize("B,Hq,Hkv,S,d,base,alpha", SMALL_BF16)
def test_bf16_shapes(env, B, Hq, Hkv, S, d, base, alpha):
    torch, oracle, atf, _ = env
    log("case: bf16 %s" % ((B, Hq, Hkv, S, d, base, alpha),))
    q, k, v, out, skipped = run_prefill(env, B, Hq, Hkv, S, d, base, alpha, torch.bfloat16)
    ref, ref_skipped = oracle.attention(q, k, v, base=base, alpha=alpha)
    dense, _ = oracle.attention(q, k, v, base=base, alpha=math.inf)
    check_bf16(out.float().cpu().numpy(), ref, dense, "bf16 %s" % ((B, Hq, Hkv, S, d),))
    assert skipped == ref_skipped
    assert skipped == B * Hq * atf.atf_skipped_pair_products(S, d, base, alpha)


@pytest.mark.parametrize("alpha", [0.5, 1.0, 2.0])
def test_bf16_high_frequency_heavy(env, alpha):
    """Fast pairs scaled x1.5: the windows change the output a lot."""
    torch, oracle, atf, _ = env
    log("case: bf16 high-frequency-heavy alpha=%g" % alpha)
    q, k, v, out, skipped = run_prefill(env, 1, 4, 1, 900, 128, 1e6, alpha, torch.bfloat16, hf=1.5)
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=alpha)
    dense, _ = oracle.attention(q, k, v, base=1e6, alpha=math.inf)
    assert np.abs(dense - ref).max() > 0.05
    check_bf16(out.float().cpu().numpy(), ref, dense, "hf alpha=%g" % alpha, structured=True)
    assert skipped == ref_skipped


@pytest.mark.parametrize("pos0", [0, 1 << 20, 1 << 24])
def test_bf16_position_shift(env, pos0):
    """Scores depend only on the distance: the kernel at pos0 matches the
    oracle at pos0 and (up to rounding) the kernel at 0."""
    torch, oracle, atf, _ = env
    log("case: bf16 pos0=%d" % pos0)
    q, k, v, out, skipped = run_prefill(env, 1, 2, 1, 500, 128, 1e6, 1.0, torch.bfloat16, pos0=pos0)
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=1.0, q_pos0=pos0, k_pos0=pos0)
    check_bf16(out.float().cpu().numpy(), ref, None, "pos0=%d" % pos0)
    out0 = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0, pos0=0)
    torch.cuda.synchronize()
    check_bf16(out.float().cpu().numpy(), out0.float().cpu().numpy(), None, "shift vs 0")
    assert skipped == ref_skipped


def test_bf16_fails_for_wrong_answers(env):
    """The checks reject a zero output and the unwindowed (dense) answer."""
    torch, oracle, atf, _ = env
    q, k, v, out, _ = run_prefill(env, 1, 2, 1, 900, 128, 1e6, 0.5, torch.bfloat16, hf=1.5)
    ref, _ = oracle.attention(q, k, v, base=1e6, alpha=0.5)
    dense, _ = oracle.attention(q, k, v, base=1e6, alpha=math.inf)
    with pytest.raises(AssertionError):
        check_bf16(np.zeros_like(ref), ref, dense, "zero", structured=True)
    with pytest.raises(AssertionError):
        check_bf16(dense, ref, dense, "dense", structured=True)
    gpu_dense = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=math.inf)
    torch.cuda.synchronize()
    with pytest.raises(AssertionError):
        check_bf16(gpu_dense.float().cpu().numpy(), ref, dense, "gpu dense", structured=True)
    check_bf16(out.float().cpu().numpy(), ref, dense, "windowed", structured=True)


@pytest.mark.parametrize("S,alpha", [(600, 0.5), (1200, 1.0)])
def test_bf16_high_frequency_x4(env, S, alpha):
    """Fast pairs scaled x4 (base 1e6, d=128): the windows move the output by
    ~5 (dense against windowed), while bf16 rounding of the rotated q and k
    alone moves it by ~0.1, beyond the fixed structured bound.  The bound is
    derived from that rounding: 3x the error of a CPU emulation whose only
    error is bf16 operands (element-wise max and per-row relative L2).  The
    result must also sit 10x closer to the windowed oracle than the dense
    answer does, and the dropped-term count is exact."""
    from bf16_emulation import emulate_bf16_operands
    torch, oracle, atf, _ = env
    log("case: bf16 x4 structured S=%d alpha=%g" % (S, alpha))
    q, k, v, out, skipped = run_prefill(env, 1, 2, 1, S, 128, 1e6, alpha, torch.bfloat16, hf=4.0)
    ref, ref_skipped = oracle.attention(q, k, v, base=1e6, alpha=alpha)
    dense, _ = oracle.attention(q, k, v, base=1e6, alpha=math.inf)
    em = emulate_bf16_operands(oracle, q.cpu(), k.cpu(), v.cpu(), 1e6, alpha)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref).max()
    em_err = np.abs(em - ref).max()
    assert err <= 3 * em_err, "max-abs %.3g > 3 x emulated bf16 error %.3g" % (err, em_err)

    def row_l2(x):
        x, r = x.reshape(-1, 128), ref.reshape(-1, 128)
        return (np.linalg.norm(x - r, axis=1) / np.linalg.norm(r, axis=1)).max()
    assert row_l2(got) <= 3 * row_l2(em)
    gap = np.abs(dense - ref).max()
    assert gap > 20 * em_err and err <= 0.1 * gap
    assert skipped == ref_skipped


def test_split_entry_points_match(env):
    """atf_prefill == atf_prefill_prepare_kv + atf_prefill_attend, bit for bit."""
    torch, oracle, atf, inputs = env
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_qkv(1, 4, 2, 513, 513, 128, dtype=torch.bfloat16, device=dev)
    a = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=1.0)
    ws = torch.empty(atf.atf_prefill_workspace_bytes(1, 2, 513, 128, atf.ATF_BF16), dtype=torch.uint8, device=dev)
    b = torch.empty_like(q)
    atf.atf_prefill_prepare_kv(k, v, rope_base=1e6, ws=ws)
    atf.atf_prefill_attend(q, k, v, b, rope_base=1e6, alpha=1.0, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def sampled_rows(Hq, S, per_head, seed, edge_tiles=0):
    """Per head: per_head seeded rows (always the first and last query) plus,
    with edge_tiles, the 256-query tile-edge rows of that many seeded tiles."""
    from rope_frequency_windowed_amd.inputs import sample_rows, tile_edge_rows
    rows = []
    for h in range(Hq):
        picked = set(int(i) for i in sample_rows(S, per_head, seed=seed + h))
        if edge_tiles:
            picked |= set(int(i) for i in tile_edge_rows(S, edge_tiles, seed=seed + 1000 + h))
        for i in sorted(picked):
            rows.append((0, h, i))
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("S,alpha,per_head,edge_tiles", [
    (32768, 1.0, 6, 1),
    (131072, 0.5, 3, 1),
    (131072, 1.0, 4, 2),
    (131072, 2.0, 3, 1),
    (1 << 20, 1.0, 4, 1),
])
def test_bf16_workload_sizes_sampled(env, S, alpha, per_head, edge_tiles):
    """The benchmark workloads (B=1, Hq=28, Hkv=4, d=128, base 1e6) in the
    launch configuration the benchmark times, checked on sampled rows of all
    28 query heads (so all 4 kv heads): always the first and last query, plus
    seeded rows and the rows at 256-query tile edges (offsets 0, 31, 32, 255:
    a workgroup's first row, the boundary of its first two waves, its last
    row), plus the exact dropped-term count."""
    torch, oracle, atf, _ = env
    B, Hq, Hkv, d, base = 1, 28, 4, 128, 1e6
    log("case: bf16 workload S=%d alpha=%g" % (S, alpha))
    q, k, v, out, skipped = run_prefill(env, B, Hq, Hkv, S, d, base, alpha, torch.bfloat16)
    assert skipped == B * Hq * atf.atf_skipped_pair_products(S, d, base, alpha)
    rows = sampled_rows(Hq, S, per_head, seed=S % 997, edge_tiles=edge_tiles)
    assert len(set(rows[:, 1].tolist())) == Hq
    sel = torch.as_tensor(rows, device=q.device)
    qrows = q[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    got = out[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    heads_kv = sorted(set(int(h) // (Hq // Hkv) for h in rows[:, 1]))
    kk = k.float().cpu().numpy()
    vv = v.float().cpu().numpy()
    del q, out
    ref, _ = oracle.attention(qrows, kk, vv, base=base, alpha=alpha, rows=rows, q_shape=(B, Hq, S, d))
    dense, _ = oracle.attention(qrows, kk, vv, base=base, alpha=math.inf, rows=rows, q_shape=(B, Hq, S, d))
    log("  kv heads %s, %d rows" % (heads_kv, len(rows)))
    assert heads_kv == list(range(Hkv))
    check_bf16(got, ref, dense, "S=%d alpha=%g" % (S, alpha))


@pytest.mark.parametrize("d,last_step_pair", [(128, 56), (256, 112)])
def test_bf16_cut_reaches_last_kstep(env, d, last_step_pair):
    """Base 1e4, alpha 0.5, S=12288: the farthest keys keep only pairs inside
    the last MFMA K-step (16 dims at d = 128, 32 dims at d = 256), so the
    kernels' last-step score chain and its in-step masking run; sampled rows
    include the last query, which sees those keys."""
    torch, oracle, atf, _ = env
    B, Hq, Hkv, S, base, alpha = 1, 4, 2, 12288, 1e4, 0.5
    W = atf.atf_window_table(d, base, alpha)
    assert W[last_step_pair - 1] < S - 1 < W[last_step_pair + 3]  # cut lands inside the last step
    log("case: last K-step d=%d S=%d" % (d, S))
    q, k, v, out, skipped = run_prefill(env, B, Hq, Hkv, S, d, base, alpha, torch.bfloat16)
    assert skipped == B * Hq * atf.atf_skipped_pair_products(S, d, base, alpha)
    rows = sampled_rows(Hq, S, 6, seed=d)
    sel = torch.as_tensor(rows, device=q.device)
    qrows = q[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    got = out[sel[:, 0], sel[:, 1], sel[:, 2]].float().cpu().numpy()
    kk, vv = k.float().cpu().numpy(), v.float().cpu().numpy()
    ref, _ = oracle.attention(qrows, kk, vv, base=base, alpha=alpha, rows=rows, q_shape=(B, Hq, S, d))
    dense, _ = oracle.attention(qrows, kk, vv, base=base, alpha=math.inf, rows=rows, q_shape=(B, Hq, S, d))
    check_bf16(got, ref, dense, "last K-step d=%d" % d)


@pytest.mark.parametrize("dtype_name", ["bfloat16", "float32"])
def test_prepared_workspace_reused(env, dtype_name):
    """One prepare, several attend calls with different alpha: each call's
    count is its own (the counter is cleared per call) and each output
    matches a fresh atf_prefill."""
    torch, oracle, atf, inputs = env
    dtype = getattr(torch, dtype_name)
    B, Hq, Hkv, S, d = 1, 4, 2, 700, 128 if dtype_name == "bfloat16" else 64
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=dtype, device=torch.device("cuda:0"))
    code = atf.ATF_BF16 if dtype_name == "bfloat16" else atf.ATF_F32
    ws = torch.empty(atf.atf_prefill_workspace_bytes(B, Hkv, S, d, code), dtype=torch.uint8, device=q.device)
    atf.atf_prefill_prepare_kv(k, v, rope_base=1e6, ws=ws)
    for alpha in (0.5, 1.0, 2.0, 1.0):
        out = torch.empty_like(q)
        got = atf.atf_prefill_attend(q, k, v, out, rope_base=1e6, alpha=alpha, ws=ws, return_skipped=True)
        assert got == B * Hq * atf.atf_skipped_pair_products(S, d, 1e6, alpha, 1, 0)
        fresh = atf.atf_prefill(q, k, v, rope_base=1e6, alpha=alpha)
        torch.cuda.synchronize()
        assert torch.equal(out, fresh)


@pytest.mark.parametrize("B,Hq,Hkv,S,d", [(1, 4, 4, 700, 128),      # plain multi-head (group 1)
                                          (1, 64, 1, 300, 64),      # the largest supported group
                                          (4, 8, 2, 257, 128)])     # a batch of sequences
def test_prefill_group_and_batch_edges(env, B, Hq, Hkv, S, d):
    torch, oracle, atf, inputs = env
    log("case: prefill edges %s" % ((B, Hq, Hkv, S, d),))
    q, k, v = inputs.make_qkv(B, Hq, Hkv, S, S, d, dtype=torch.bfloat16, device=torch.device("cuda:0"))
    out, skipped = atf.atf_prefill(q, k, v, rope_base=1e4, alpha=1.0, return_skipped=True)
    torch.cuda.synchronize()
    ref, ref_skipped = oracle.attention(q, k, v, base=1e4, alpha=1.0)
    check_bf16(out.float().cpu().numpy(), ref, None, "prefill edges")
    assert skipped == ref_skipped
