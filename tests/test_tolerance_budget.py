"""Sizes the bf16 parity bound on the CPU: emulates a kernel whose only error
is bf16 rounding of its operands (rotated q and k, probabilities, values; all
products and sums exact) and checks that this inherent error sits well inside
the bounds the GPU parity tests use, for the iid inputs and for the
structured (fast pairs x1.5) inputs."""
import numpy as np
import pytest
import torch

from bf16_emulation import emulate_bf16_operands
from parity import BF16_ATOL
from rope_frequency_windowed_amd.inputs import make_qkv


@pytest.mark.parametrize("hf", [None, 1.5])
@pytest.mark.parametrize("alpha", [0.5, 1.0])
def test_bf16_rounding_fits_the_bound(orc, hf, alpha):
    q, k, v = make_qkv(1, 2, 1, 600, 600, 128, dtype=torch.bfloat16, high_freq_scale=hf)
    ref, _ = orc.attention(q, k, v, base=1e6, alpha=alpha)
    em = emulate_bf16_operands(orc, q, k, v, 1e6, alpha)
    err, scale = np.abs(em - ref).max(), np.abs(ref).max()
    bound = BF16_ATOL * (max(1.0, scale) if hf else 1.0)
    assert err <= 0.5 * bound
    assert err <= 0.5 * 1e-2 * scale


@pytest.mark.parametrize("S,alpha", [(600, 0.5), (1200, 1.0)])
def test_x4_inputs_need_the_derived_bound(orc, S, alpha):
    """Fast pairs x4: bf16 operand rounding alone exceeds the fixed structured
    bound (so the GPU test of these inputs is held to a bound derived from
    this emulation instead), while the windows move the output by more than
    20x that rounding error (so the case still tells windowed from dense)."""
    import math
    q, k, v = make_qkv(1, 2, 1, S, S, 128, dtype=torch.bfloat16, high_freq_scale=4.0)
    ref, _ = orc.attention(q, k, v, base=1e6, alpha=alpha)
    dense, _ = orc.attention(q, k, v, base=1e6, alpha=math.inf)
    em = emulate_bf16_operands(orc, q, k, v, 1e6, alpha)
    err, scale = np.abs(em - ref).max(), np.abs(ref).max()
    assert err > 0.9 * BF16_ATOL * max(1.0, scale)
    assert np.abs(dense - ref).max() > 20 * err
