"""CPU emulation of a kernel whose only error is bf16 rounding of its
operands (rotated q and k, probabilities, values), with every product and sum
exact (fp64).  Sizes the bf16 parity bounds (not a test module)."""
import math

import numpy as np
import torch

from oracle import dense_ref


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def emulate_bf16_operands(orc, q, k, v, base, alpha):
    q, k, v = (t.double().numpy() for t in (q, k, v))
    S, d = q.shape[2], q.shape[3]
    P = d // 2
    W = orc.window_table(d, base, alpha).astype(np.float64)
    W[orc.window_table(d, base, alpha) == orc.W_INF] = np.inf
    pos = np.arange(S)
    qr = bf16(dense_ref.rope_half_split(q, pos, base))
    kr = np.repeat(bf16(dense_ref.rope_half_split(k, pos, base)), q.shape[1] // k.shape[1], 1)
    vv = np.repeat(v, q.shape[1] // k.shape[1], 1)
    delta = pos[:, None] - pos[None, :]
    s = np.zeros(q.shape[:2] + (S, S))
    for p in range(P):
        t = (qr[..., p][..., :, None] * kr[..., p][..., None, :]
             + qr[..., p + P][..., :, None] * kr[..., p + P][..., None, :])
        s += np.where(delta <= W[p], t, 0.0)
    lg = np.where(delta >= 0, s / math.sqrt(d), -np.inf)
    w = bf16(np.exp(lg - lg.max(-1, keepdims=True)))
    return (w @ vv) / w.sum(-1, keepdims=True)
