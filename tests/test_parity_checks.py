"""The GPU parity checks themselves, on the CPU: a correct result passes, and
results a broken kernel would give (the dense answer, a blend of dense and
windowed, zeros) fail.  Parity helpers live in tests/parity.py."""
import math

import numpy as np
import pytest
import torch

from parity import check_bf16
from rope_frequency_windowed_amd.inputs import make_qkv


def _bf16_round(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


@pytest.fixture(scope="module")
def windowed_and_dense(orc):
    # fast pairs x1.5: the windows move the output far beyond the bf16 bound
    q, k, v = make_qkv(1, 2, 1, 300, 300, 64, dtype=torch.bfloat16, high_freq_scale=1.5)
    ref, _ = orc.attention(q, k, v, base=1e4, alpha=0.5)
    dense, _ = orc.attention(q, k, v, base=1e4, alpha=math.inf)
    assert np.abs(dense - ref).max() > 0.1
    return ref, dense


def test_correct_result_passes(windowed_and_dense):
    ref, dense = windowed_and_dense
    check_bf16(_bf16_round(ref), ref, dense, "bf16-rounded oracle", structured=True)


def test_dense_result_fails(windowed_and_dense):
    ref, dense = windowed_and_dense
    with pytest.raises(AssertionError):
        check_bf16(dense, ref, dense, "dense as the result", structured=True)


def test_zero_result_fails(windowed_and_dense):
    ref, dense = windowed_and_dense
    with pytest.raises(AssertionError):
        check_bf16(np.zeros_like(ref), ref, dense, "zeros", structured=True)


def _blend_case():
    # max|ref| = 1: the bf16 bound is min(2e-2, 1e-2 * 1) = 1e-2; the windows
    # move one element by 0.06 (> 4x the bound)
    ref = np.full((4, 64), 0.5)
    ref[0, 0] = 1.0
    dense = ref.copy()
    dense[1, 3] += 0.06
    return ref, dense


def test_discrimination_alone_catches_a_blend():
    """15% of the dense answer mixed in: inside every max-abs and row bound,
    caught only by the discrimination check."""
    ref, dense = _blend_case()
    blend = ref + 0.15 * (dense - ref)
    check_bf16(blend, ref, None, "blend without dense")  # the other bounds pass
    with pytest.raises(AssertionError, match="not discriminating"):
        check_bf16(blend, ref, dense, "blend")


def test_discrimination_accepts_small_error():
    ref, dense = _blend_case()
    noisy = ref + 0.04 * (dense - ref)
    check_bf16(noisy, ref, dense, "4% of the gap")


def test_discrimination_inactive_when_windows_do_not_matter():
    """When dense and windowed agree to within the bound, a correct result is
    not asked to beat the bf16 rounding."""
    ref = np.full((2, 64), 0.5)
    ref[0, 0] = 1.0
    dense = ref.copy()
    dense[1, 3] += 0.01  # 1x the bound
    check_bf16(ref + 0.5 * (dense - ref), ref, dense, "windows below the bound")
