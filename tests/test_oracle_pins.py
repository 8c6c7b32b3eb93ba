"""Pins for the fp64 oracle: things the source page and plain mathematics fix,
none of which re-types the oracle's own formula.

Source page for the method: "ATFlash: RoPE-Frequenzen kuerzen
Attention-Arbeit um bis zu 57 Prozent" (sudo-ai.de):
  * section "Was ATFlash anders macht": per-pair windows proportional to the
    wavelength; fast pairs drop out first; distant keys stay reachable through
    the slow pairs;
  * section "Die Zahlen - und ihre Grenze": the online softmax is unchanged.
"""
import math
import os

import numpy as np
import pytest

from oracle import dense_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


# ----------------------------------------------------------------- window table

def test_window_closed_forms(orc):
    """Hand-derived W_p at pairs whose wavelength is 2*pi*10^k."""
    n = 0
    with open(os.path.join(GOLDEN, "window_closed_forms.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            d, base, alpha, p, w = line.split()
            W = orc.window_table(int(d), float(base), float(alpha))
            expect = orc.W_INF if w == "inf" else int(w)
            assert W[int(p)] == expect, line
            n += 1
    assert n >= 20


@pytest.mark.parametrize("d,base", [(64, 1e4), (128, 1e6), (128, 1e4), (16, 10.0), (256, 1e6), (256, 1e4)])
@pytest.mark.parametrize("alpha", [0.25, 0.5, 1.0, 2.0, 7.5])
def test_window_structure(orc, d, base, alpha):
    W = orc.window_table(d, base, alpha)
    assert W.shape == (d // 2,)
    assert W[-1] == orc.W_INF                      # slowest pair never cut
    assert np.all(np.diff(W) >= 0)                 # fast pairs are cut first
    assert W[0] == math.ceil(2 * math.pi * alpha)  # theta_0 = 1
    assert np.all(W[:-1] > 0)


def test_window_alpha_inf(orc):
    W = orc.window_table(128, 1e6, math.inf)
    assert np.all(W == orc.W_INF)


def test_window_rejects_bad_args(orc):
    for args in [(63, 1e4, 1.0), (64, 1.0, 1.0), (64, 1e4, 0.0), (64, 1e4, -1.0),
                 (64, 1e4, float("nan"))]:
        with pytest.raises(ValueError):
            orc.window_table(*args)


@pytest.mark.parametrize("d,base,alpha", [(64, 1e4, 1.0), (128, 1e6, 0.5), (128, 1e6, 1.0),
                                          (128, 1e6, 2.0)])
def test_window_margin_at_workloads(d, base, alpha):
    """alpha*lambda_p sits far from an integer at every benchmarked setting, so
    any fp64 evaluation order gives the same ceiling (a float32 one would not)."""
    margins = []
    for p in range(d // 2 - 1):
        x = alpha * 2 * math.pi * base ** (2 * p / d)
        margins.append(abs(x - round(x)))
    assert min(margins) > 1e-6


# ---------------------------------------------------------------- skipped count

def brute_force_count(W, q_pos, k_pos, causal=True):
    """Enumerate every (query, key, pair) and count dropped terms."""
    delta = q_pos[:, None] - k_pos[None, :]
    live = delta >= 0 if causal else np.ones_like(delta, dtype=bool)
    dist = delta if causal else np.abs(delta)
    total = 0
    for w in W:
        if w == np.iinfo(np.int64).max:
            continue
        total += int(np.sum(live & (dist > w)))
    return total


@pytest.mark.parametrize("S,d,base,alpha", [(64, 16, 10.0, 0.3), (200, 16, 10.0, 1.0),
                                            (256, 64, 1e4, 1.0), (97, 32, 100.0, 0.7),
                                            (2048, 64, 1e4, 1.0), (1500, 128, 1e6, 0.5),
                                            (3000, 256, 1e4, 1.0)])
def test_count_closed_form_equals_brute_force(orc, S, d, base, alpha):
    W = orc.window_table(d, base, alpha)
    pos = np.arange(S)
    bf = brute_force_count(W, pos, pos)
    assert orc.skipped_closed_form(S, d, base, alpha) == bf
    # decode geometry: one query after S keys
    bf_dec = brute_force_count(W, np.array([S]), pos)
    assert orc.skipped_closed_form(S, d, base, alpha, decode=True) == bf_dec


def test_count_small_config_value(orc):
    """S=256, d=64, base 1e4, alpha 1 (the fp32 parity workload): brute force."""
    W = orc.window_table(64, 1e4, 1.0)
    pos = np.arange(256)
    bf = brute_force_count(W, pos, pos)
    assert bf == orc.skipped_closed_form(256, 64, 1e4, 1.0)
    with open(os.path.join(GOLDEN, "count_s256_d64.txt")) as f:
        stored = int([l for l in f if not l.startswith("#")][0])
    assert bf == stored


@pytest.mark.parametrize("causal", [True, False])
def test_oracle_enumerated_count_matches(orc, causal):
    """The count the attention loop itself accumulates equals the brute force."""
    B, Hq, Hkv, S, d = 2, 4, 2, 150, 32
    q, k, v = rnd((B, Hq, S, d), 1), rnd((B, Hkv, S, d), 2), rnd((B, Hkv, S, d), 3)
    _, skipped = orc.attention(q, k, v, base=100.0, alpha=0.5, causal=causal)
    W = orc.window_table(d, 100.0, 0.5)
    pos = np.arange(S)
    assert skipped == B * Hq * brute_force_count(W, pos, pos, causal=causal)
    if causal:
        assert skipped == B * Hq * orc.skipped_closed_form(S, d, 100.0, 0.5)


def test_count_monotone_and_limits(orc):
    S, d, base = 4096, 128, 1e6
    counts = [orc.skipped_closed_form(S, d, base, a) for a in (0.25, 0.5, 1, 2, 4, 16)]
    assert all(a >= b for a, b in zip(counts, counts[1:]))
    assert orc.skipped_closed_form(S, d, base, math.inf) == 0
    W0 = int(orc.window_table(d, base, 1.0)[0])
    assert orc.skipped_closed_form(W0 + 1, d, base, 1.0) == 0
    assert orc.skipped_closed_form(W0 + 2, d, base, 1.0) == 1


# -------------------------------------------------------- reductions to textbook

@pytest.mark.parametrize("causal", [True, False])
def test_alpha_inf_equals_dense(orc, causal):
    B, Hq, Hkv, S, d = 2, 6, 2, 70, 32
    q, k, v = rnd((B, Hq, S, d), 11), rnd((B, Hkv, S, d), 12), rnd((B, Hkv, S, d), 13)
    out, skipped = orc.attention(q, k, v, base=1e4, alpha=math.inf, causal=causal, q_pos0=5, k_pos0=5)
    ref = dense_ref.dense_rope_attention(q, k, v, base=1e4, causal=causal, q_pos0=5, k_pos0=5)
    assert skipped == 0
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


def test_alpha_inf_equals_dense_d256(orc):
    """d = 256 (128 pairs, more than a wave's 64 lanes on the GPU side)."""
    B, Hq, Hkv, S, d = 1, 2, 1, 60, 256
    q, k, v = rnd((B, Hq, S, d), 14), rnd((B, Hkv, S, d), 15), rnd((B, Hkv, S, d), 16)
    out, skipped = orc.attention(q, k, v, base=1e4, alpha=math.inf)
    ref = dense_ref.dense_rope_attention(q, k, v, base=1e4)
    assert skipped == 0
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


def test_alpha_inf_decode_equals_dense(orc):
    B, Hq, Hkv, S, d = 3, 4, 2, 90, 64
    q, k, v = rnd((B, Hq, 1, d), 21), rnd((B, Hkv, S, d), 22), rnd((B, Hkv, S, d), 23)
    out, _ = orc.attention(q, k, v, base=1e6, alpha=math.inf, q_pos0=S + 3, k_pos0=3)
    ref = dense_ref.dense_rope_attention(q, k, v, base=1e6, q_pos0=S + 3, k_pos0=3)
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


def test_short_sequence_equals_dense(orc):
    """All distances <= W_0: no pair is ever cut."""
    W0 = int(orc.window_table(64, 1e4, 1.0)[0])
    S = W0 + 1
    q, k, v = rnd((1, 2, S, 64), 31), rnd((1, 2, S, 64), 32), rnd((1, 2, S, 64), 33)
    out, skipped = orc.attention(q, k, v, base=1e4, alpha=1.0)
    ref = dense_ref.dense_rope_attention(q, k, v, base=1e4)
    assert skipped == 0
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("alpha", [0.1, 1.0, 3.0])
def test_slowest_pair_only_equals_dense(orc, alpha):
    """Inputs living only on the never-cut pair P-1 see no window at all."""
    S, d = 300, 32
    P = d // 2
    q, k, v = rnd((1, 1, S, d), 41), rnd((1, 1, S, d), 42), rnd((1, 1, S, d), 43)
    mask = np.zeros(d, dtype=np.float32)
    mask[[P - 1, d - 1]] = 1.0
    q, k = q * mask, k * mask
    out, _ = orc.attention(q, k, v, base=100.0, alpha=alpha)
    ref = dense_ref.dense_rope_attention(q, k, v, base=100.0)
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


def explicit_single_pair(q, k, v, p, base, W_p, q_pos, k_pos, causal=True):
    """Attention when q and k live only on pair p, built from the
    relative-angle identity (no rotation of vectors at all):
      score = (q_lo k_lo + q_hi k_hi) cos(delta*theta) + (q_lo k_hi - q_hi k_lo) sin(delta*theta)
    kept iff distance <= W_p; logits = score / sqrt(d)."""
    d = q.shape[-1]
    P = d // 2
    theta = base ** (-2.0 * p / d)
    ql, qh = q[:, p].astype(np.float64), q[:, p + P].astype(np.float64)
    kl, kh = k[:, p].astype(np.float64), k[:, p + P].astype(np.float64)
    delta = (q_pos[:, None] - k_pos[None, :]).astype(np.float64)
    A = ql[:, None] * kl[None, :] + qh[:, None] * kh[None, :]
    Bs = ql[:, None] * kh[None, :] - qh[:, None] * kl[None, :]
    score = A * np.cos(delta * theta) + Bs * np.sin(delta * theta)
    dist = delta if causal else np.abs(delta)
    score = np.where(dist <= W_p, score, 0.0)
    logits = score / math.sqrt(d)
    if causal:
        logits = np.where(delta >= 0, logits, -np.inf)
    logits -= logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=1, keepdims=True)
    return w @ v.astype(np.float64)


@pytest.mark.parametrize("p", [0, 3, 7, 12, 15])
@pytest.mark.parametrize("causal", [True, False])
def test_single_pair_explicit_logits(orc, p, causal):
    """Pins the pair layout (p, p+P), the rotation sign, the inclusive window
    (distance <= W_p), the zero (not -inf) value of a dropped term and the
    1/sqrt(d) scale, all at once."""
    S, d, base, alpha = 260, 32, 20.0, 0.8
    P = d // 2
    q, k, v = rnd((1, 1, S, d), 50 + p), rnd((1, 1, S, d), 60 + p), rnd((1, 1, S, d), 70 + p)
    mask = np.zeros(d, dtype=np.float32)
    mask[[p, p + P]] = 1.0
    q, k = q * mask, k * mask
    W = orc.window_table(d, base, alpha)
    assert W[p] < S - 1 or p == P - 1  # the window really cuts inside this sequence
    out, _ = orc.attention(q, k, v, base=base, alpha=alpha, causal=causal, q_pos0=9, k_pos0=9)
    pos = 9 + np.arange(S)
    Wp = np.inf if W[p] == orc.W_INF else float(W[p])
    ref = explicit_single_pair(q[0, 0], k[0, 0], v[0, 0], p, base, Wp, pos, pos, causal)
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-11, rtol=0)


def test_single_pair_decode_geometry(orc):
    S, d, base, alpha, p = 500, 16, 10.0, 1.0, 2
    P = d // 2
    q, k, v = rnd((1, 1, 1, d), 81), rnd((1, 1, S, d), 82), rnd((1, 1, S, d), 83)
    mask = np.zeros(d, dtype=np.float32)
    mask[[p, p + P]] = 1.0
    q, k = q * mask, k * mask
    W = orc.window_table(d, base, alpha)
    out, skipped = orc.attention(q, k, v, base=base, alpha=alpha, q_pos0=S, k_pos0=0)
    ref = explicit_single_pair(q[0, 0], k[0, 0], v[0, 0], p, base, float(W[p]),
                               np.array([S]), np.arange(S))
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-11, rtol=0)
    assert skipped == orc.skipped_closed_form(S, d, base, alpha, decode=True)


# ------------------------------------------------------ GPT-J interleaved pairs

def halfsplit_of_interleaved(x):
    """Dims (2p, 2p+1) of each row moved to (p, p+P): the half-split row that
    carries the same rotary pairs."""
    x = np.asarray(x)
    return np.concatenate([x[..., 0::2], x[..., 1::2]], axis=-1)


@pytest.mark.parametrize("causal", [True, False])
def test_gptj_alpha_inf_equals_dense(orc, causal):
    """Windows off: the interleaved layout equals dense attention whose rotary
    is the complex-number rotation of (x_2p + i x_2p+1)."""
    B, Hq, Hkv, S, d = 1, 4, 2, 75, 32
    q, k, v = rnd((B, Hq, S, d), 151), rnd((B, Hkv, S, d), 152), rnd((B, Hkv, S, d), 153)
    out, skipped = orc.attention(q, k, v, base=1e4, alpha=math.inf, causal=causal, q_pos0=7, k_pos0=7,
                                 layout="gptj")
    ref = dense_ref.dense_rope_attention(q, k, v, base=1e4, causal=causal, q_pos0=7, k_pos0=7, layout="gptj")
    assert skipped == 0
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("alpha", [0.3, 1.0])
def test_gptj_equals_halfsplit_on_moved_dims(orc, alpha):
    """Pair p is the same pair in both layouts, only stored elsewhere: moving
    q's and k's dims (2p, 2p+1) to (p, p+P) gives the half-split result
    exactly, windows and count included (values are not rotary, not moved)."""
    B, Hq, Hkv, S, d = 2, 4, 2, 140, 32
    q, k, v = rnd((B, Hq, S, d), 161), rnd((B, Hkv, S, d), 162), rnd((B, Hkv, S, d), 163)
    a, sa = orc.attention(q, k, v, base=50.0, alpha=alpha, layout="gptj")
    b, sb = orc.attention(halfsplit_of_interleaved(q), halfsplit_of_interleaved(k), v, base=50.0, alpha=alpha)
    assert sa == sb > 0
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("p", [0, 5, 15])
def test_gptj_single_pair_explicit_logits(orc, p):
    """q, k on dims (2p, 2p+1) only: the relative-angle formula with a cut
    window, written for that pair."""
    S, d, base, alpha = 240, 32, 20.0, 0.8
    q, k, v = rnd((1, 1, S, d), 170 + p), rnd((1, 1, S, d), 180 + p), rnd((1, 1, S, d), 190 + p)
    mask = np.zeros(d, dtype=np.float32)
    mask[[2 * p, 2 * p + 1]] = 1.0
    q, k = q * mask, k * mask
    W = orc.window_table(d, base, alpha)
    out, _ = orc.attention(q, k, v, base=base, alpha=alpha, q_pos0=4, k_pos0=4, layout="gptj")
    pos = 4 + np.arange(S)
    Wp = np.inf if W[p] == orc.W_INF else float(W[p])
    ref = explicit_single_pair(halfsplit_of_interleaved(q[0, 0]), halfsplit_of_interleaved(k[0, 0]), v[0, 0], p,
                               base, Wp, pos, pos)
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-11, rtol=0)


def test_gptj_shift_invariance(orc):
    B, Hq, Hkv, S, d = 1, 2, 1, 100, 64
    q, k, v = rnd((B, Hq, S, d), 201), rnd((B, Hkv, S, d), 202), rnd((B, Hkv, S, d), 203)
    a, sa = orc.attention(q, k, v, base=1e4, alpha=1.0, layout="gptj")
    b, sb = orc.attention(q, k, v, base=1e4, alpha=1.0, q_pos0=2 ** 22, k_pos0=2 ** 22, layout="gptj")
    assert sa == sb
    np.testing.assert_allclose(a, b, atol=1e-9, rtol=0)


def test_layout_name_checked(orc):
    q = rnd((1, 1, 4, 8), 1)
    with pytest.raises(ValueError):
        orc.attention(q, q, q, base=1e4, alpha=1.0, layout="interleaved")


# ------------------------------------------------------------------ invariances

@pytest.mark.parametrize("shift", [2 ** 20, 2 ** 24 + 3])
def test_shift_invariance(orc, shift):
    """Scores depend only on the distance, so moving every position by the same
    amount leaves the output unchanged."""
    B, Hq, Hkv, S, d = 1, 2, 1, 120, 64
    q, k, v = rnd((B, Hq, S, d), 91), rnd((B, Hkv, S, d), 92), rnd((B, Hkv, S, d), 93)
    a, sa = orc.attention(q, k, v, base=1e4, alpha=1.0)
    b, sb = orc.attention(q, k, v, base=1e4, alpha=1.0, q_pos0=shift, k_pos0=shift)
    assert sa == sb
    np.testing.assert_allclose(a, b, atol=1e-9, rtol=0)


def test_gqa_equals_repeated_heads(orc):
    B, Hq, Hkv, S, d = 2, 6, 2, 80, 32
    q, k, v = rnd((B, Hq, S, d), 101), rnd((B, Hkv, S, d), 102), rnd((B, Hkv, S, d), 103)
    a, _ = orc.attention(q, k, v, base=1e4, alpha=0.5)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    b, _ = orc.attention(q, kr, vr, base=1e4, alpha=0.5)
    np.testing.assert_array_equal(a, b)


def test_every_causal_key_reachable(orc):
    """One-hot values read the softmax weights back: every key at or before the
    query keeps a positive weight (the slow pair still sees it), later keys get
    exactly zero."""
    S = d = 64
    q, k = rnd((1, 1, S, d), 111) * 3, rnd((1, 1, S, d), 112) * 3
    v = np.eye(S, dtype=np.float32)[None, None]
    out, _ = orc.attention(q, k, v, base=1e4, alpha=0.05)  # tiny windows: almost all cut
    w = out[0, 0]
    i, j = np.indices((S, S))
    assert np.all(w[j <= i] > 0)
    assert np.all(w[j > i] == 0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-12)


def test_rows_subset_matches_full(orc):
    B, Hq, Hkv, S, d = 2, 4, 2, 64, 32
    q, k, v = rnd((B, Hq, S, d), 121), rnd((B, Hkv, S, d), 122), rnd((B, Hkv, S, d), 123)
    full, _ = orc.attention(q, k, v, base=1e4, alpha=1.0)
    rows = np.array([[0, 0, 0], [1, 3, 63], [0, 2, 17], [1, 1, 40]])
    sub, _ = orc.attention(q, k, v, base=1e4, alpha=1.0, rows=rows)
    for r, (b, h, i) in enumerate(rows):
        np.testing.assert_array_equal(sub[r], full[b, h, i])


def test_compact_query_rows_match_full(orc):
    B, Hq, Hkv, S, d = 1, 4, 1, 90, 32
    q, k, v = rnd((B, Hq, S, d), 141), rnd((B, Hkv, S, d), 142), rnd((B, Hkv, S, d), 143)
    rows = np.array([[0, 3, 89], [0, 0, 0], [0, 2, 45]])
    full, sf = orc.attention(q, k, v, base=1e4, alpha=0.7, rows=rows)
    qc = np.stack([q[b, h, i] for b, h, i in rows])
    comp, sc = orc.attention(qc, k, v, base=1e4, alpha=0.7, rows=rows, q_shape=q.shape)
    np.testing.assert_array_equal(full, comp)
    assert sf == sc


def test_windows_change_the_output(orc):
    """A discrimination check: at a short window the windowed output differs
    clearly from dense attention."""
    S, d = 200, 32
    q, k, v = rnd((1, 1, S, d), 131), rnd((1, 1, S, d), 132), rnd((1, 1, S, d), 133)
    a, _ = orc.attention(q, k, v, base=100.0, alpha=0.5)
    b, _ = orc.attention(q, k, v, base=100.0, alpha=math.inf)
    assert np.max(np.abs(a - b)) > 0.05


def _chunk_closed_form(Sq, Sk, W):
    """Dropped (query, key, pair) terms of one head when Sq queries sit at key
    indices Sk-Sq .. Sk-1: query at index t drops pair p for the t - W_p keys
    farther than W_p, so the count is F(Sk-1) - F(Sk-Sq-1) with
    F(T) = sum_p n(n+1)/2, n = max(0, T - W_p)."""
    def F(T):
        tot = 0
        for w in W:
            if w == np.iinfo(np.int64).max:
                continue
            n = max(0, T - int(w))
            tot += n * (n + 1) // 2
        return tot
    return F(Sk - 1) - F(Sk - Sq - 1)


@pytest.mark.parametrize("Sq,Sk", [(1, 40), (7, 40), (40, 40), (13, 100)])
def test_chunk_equals_last_rows_of_full_prefill(orc, Sq, Sk):
    """A chunk of Sq queries after Sk-Sq cached tokens is the last Sq rows of
    the full causal prefill over Sk tokens, and its dropped-term count has the
    closed form above (brute-force enumeration by the oracle)."""
    d, base, alpha = 16, 10.0, 1.0
    q = rnd((1, 2, Sk, d), 11)
    k = rnd((1, 1, Sk, d), 12)
    v = rnd((1, 1, Sk, d), 13)
    full, _ = orc.attention(q, k, v, base=base, alpha=alpha, q_pos0=5, k_pos0=5)
    qc = np.ascontiguousarray(q[:, :, Sk - Sq:, :])
    part, cnt = orc.attention(qc, k, v, base=base, alpha=alpha, q_pos0=5 + Sk - Sq, k_pos0=5)
    np.testing.assert_allclose(part, full[:, :, Sk - Sq:, :], rtol=0, atol=1e-12)
    W = orc.window_table(d, base, alpha)
    assert cnt == 2 * _chunk_closed_form(Sq, Sk, W)
